"""Nested (double-quantized) 4-bit state: encode and fused-scale dequantize.

Test infrastructure only.

Dequantize follows [PR2051] Summary and Implementation: the per-block fp32
scale is rebuilt from an 8-bit dynamic-map code, the fp32 absmax of its group
of 256 blocks and a mean offset, as a separately rounded multiply and then a
separately rounded add (no fused multiply-add); the 4-bit values are then
decoded with that scale exactly as in the plain path:

    s_b   = RN( RN(qmap2[code_b] * absmax2[floor(b / 256)]) + offset )
    out_e = RN_T( RN(c[idx_e] * s_{floor(e / B)}) )

Encode is not on the pages (the configuration text says "per-block absmax
minus its mean offset is 8-bit dynamic-map quantized in groups of 256").
Reading used here:

    offset    = RN32( (sum of a_b, exact) / nb ): the mean, rounded once to
                fp32 (0 for nb = 0; NaN if any a_b is NaN or both infinities
                occur; +-inf if one infinity occurs)
    r_b       = RN(a_b - offset)
    (code, absmax2) = blockwise quantize of r with block 256 and the dynamic
                      map as codebook (the same first-index nearest rule, the
                      same 1e-8 clamp; the last group may be short).

Parity: dequantize is pinned in ``tests/test_oracle_nested.py`` (reduction to
the plain path when offset = 0 and absmax2 = 1; an FMA canary whose fused
result differs from the separately rounded one, checked with exact
rationals).  Encode is pinned in the same file: the offset against exact
rational means (including sums that fp32 or fp64 accumulation gets wrong),
the rest against the definition written with exact rationals, and the
round-trip error bound.
"""

import numpy as np

from . import kbit
from .numerics import exact_sum_f32, narrow, rn32_rational

GROUP2 = 256


def mean_offset(a):
    """RN32 of the exact mean of fp32 values (see the reading above)."""
    a = np.asarray(a, dtype=np.float32).ravel()
    if a.size == 0:
        return np.float32(0.0)
    if np.isnan(a).any() or (np.isposinf(a).any() and np.isneginf(a).any()):
        return np.float32(np.nan)
    if np.isposinf(a).any():
        return np.float32(np.inf)
    if np.isneginf(a).any():
        return np.float32(-np.inf)
    return rn32_rational(exact_sum_f32(a), a.size << 149)


def encode(absmax, qmap2):
    """Nested state for fp32 per-block absmax: (code u8, absmax2 f32, offset f32)."""
    a = np.asarray(absmax, dtype=np.float32).ravel()
    nb = a.size
    if nb == 0:
        return np.zeros(0, np.uint8), np.zeros(0, np.float32), np.float32(0.0)
    offset = mean_offset(a)
    with np.errstate(invalid="ignore", over="ignore"):
        r = (a - offset).astype(np.float32)
    code, absmax2 = kbit.quantize(r, qmap2, GROUP2)
    return code, absmax2, offset


def scales(code, absmax2, offset, qmap2):
    """s_b = RN(RN(qmap2[code_b] * absmax2[b // 256]) + offset)."""
    code = np.asarray(code, dtype=np.uint8).ravel()
    q = np.asarray(qmap2, dtype=np.float32)[code]
    g = np.arange(code.size, dtype=np.int64) // GROUP2
    prod = (q * np.asarray(absmax2, dtype=np.float32)[g]).astype(np.float32)
    return (prod + np.float32(offset)).astype(np.float32)


def dequantize(idx, code, absmax2, offset, qmap2, codebook, B, out_dtype):
    s = scales(code, absmax2, offset, qmap2)
    return narrow(kbit.dequantize_values(idx, s, codebook, B), out_dtype)


def dequantize_packed(words, code, absmax2, offset, qmap2, codebook, n, B, out_dtype):
    idx = kbit.unpack(words, 4, n)
    return dequantize(idx, code, absmax2, offset, qmap2, codebook, B, out_dtype)
