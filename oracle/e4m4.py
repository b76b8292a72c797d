"""E4M4 uint8 block scales: encode, decode, and the k-bit paths that use them.

Test infrastructure only.  Follows [QLORA-2] PATCH 005 "Add vectorized
dequant kernel and E4M4 uint8 absmax" (``functional.py``
``encode_absmax_e4m4`` / ``decode_absmax_e4m4``, the kernel-side decoder, and
``quantize_kbit(..., absmax_format="e4m4")``):

* Format: byte = e << 4 | m with bias 11.
  e > 0: 2^(e - 11) * (1 + m/16); e = 0: 2^(1 - 11) * m/16 (so 0x00 is 0).
* Encode, for a > 0 (other values give 0):
    e_u = floor(log2 a);  e_b = clamp(e_u + 11, 0, 15);
    e_u + 11 <= 0  ->  subnormal: e_b = 0, m = rne(a / 2^(1-11) * 16)
    otherwise          m = rne((a / 2^e_u - 1) * 16)
    m clamped to [0, 15] (rne = round half to even, as torch.round).
  Reading: floor(log2 a) is taken exactly (the binary exponent of a); the
  page evaluates log2 in float32, which can round a value just below a power
  of two up to it.  Above the range (e_u + 11 > 15) the page keeps e_b = 15
  with the mantissa of the unclamped exponent; so does this module.
  Non-finite scales are outside the format and the page leaves them open:
  NaN fails the page's a > 0 test and gives 0; +inf is read as exponent 15
  with mantissa 0 (its exponent is above the range, its fraction bits are 0).
* quantize_kbit with E4M4: indices come from the fp32 absmax exactly as in
  the fp32 path; only the stored scale is encoded.
* dequantize: out = RN_T(RN(c[idx] * decode(code_b))).

Every step is exact integer or power-of-two arithmetic in float64 except
the final product, which is rounded to fp32 as in the fp32 path.

Parity: pinned in ``tests/test_oracle_e4m4.py`` (all 256 codes decoded with
exact rationals; encode(decode(c)) == c for every code; nearest-in-grid
with ties to even; the page's round-trip test values).
"""

import numpy as np

from . import kbit
from .numerics import narrow

BIAS = 11


def decode(code, bias=BIAS):
    """uint8 codes -> float32 scales."""
    c = np.asarray(code).astype(np.int64)
    e = c >> 4
    m = (c & 0xF).astype(np.float64)
    out = np.where(e == 0, np.ldexp(m / 16.0, 1 - bias), np.ldexp(1.0 + m / 16.0, e - bias))
    return out.astype(np.float32)


def encode(a, bias=BIAS):
    """float32 scales -> uint8 codes."""
    a = np.asarray(a, dtype=np.float32)
    out = np.zeros(a.shape, dtype=np.uint8)
    inf = np.isposinf(a)
    nz = (a > 0) & ~inf                          # NaN and non-positive give 0
    v = a[nz].astype(np.float64)
    frac, exp = np.frexp(v)                      # v = frac * 2^exp, frac in [0.5, 1)
    e_u = exp.astype(np.int64) - 1               # floor(log2 v), exact
    sub = (e_u + bias) <= 0
    e_b = np.clip(e_u + bias, 0, 15)
    e_b[sub] = 0
    m_norm = np.rint((np.ldexp(v, -e_u) - 1.0) * 16.0)       # exact argument; rint = half to even
    m_sub = np.rint(np.ldexp(v, -(1 - bias)) * 16.0)
    m = np.where(sub, m_sub, m_norm)
    m = np.clip(m, 0, 15).astype(np.int64)
    out[nz] = ((e_b << 4) | m).astype(np.uint8)
    out[inf] = 0xF0
    return out


def quantize_packed(x, codebook, K, B):
    """k-bit quantize with E4M4 scales: (words, codes)."""
    words, absmax = kbit.quantize_packed(x, codebook, K, B)
    return words, encode(absmax)


def dequantize(idx, code, codebook, B, out_dtype):
    """out = RN_T(RN(c[idx] * decode(code_b)))."""
    return narrow(kbit.dequantize_values(idx, decode(code), codebook, B), out_dtype)
