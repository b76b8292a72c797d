"""Element formats used by the oracle (test infrastructure only).

bf16 tensors are carried as ``np.uint16`` raw bit patterns (numpy has no
bfloat16); fp16 tensors as ``np.float16``; fp32 as ``np.float32``.

* widening bf16/fp16 -> fp32 is exact ([QLORA-2] PATCH 001, ``csrc/kernels.cu``
  ``kQuantizeBlockwise_kbit`` step 1 converts the element to float before any
  arithmetic);
* narrowing fp32 -> bf16/fp16 rounds to nearest, ties to even, keeps gradual
  underflow and signed zeros ([QLORA-2] PATCH 001 ``kDequantizeBlockwise_kbit``
  step 7 casts the fp32 product to the output type; ``dequantize_kbit_ref``
  ends with ``.to(dtype)``).  NaN inputs are out of scope.

Parity: pinned in ``tests/test_oracle_numerics.py`` against exact rational
rounding written with ``fractions.Fraction``.
"""

import numpy as np

F32 = np.float32

DTYPES = ("fp32", "fp16", "bf16")


def widen(a, dtype):
    """Exact conversion of a bf16/fp16/fp32 array to float32."""
    if dtype == "bf16":
        a = np.asarray(a, dtype=np.uint16)
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32)
    if dtype == "fp16":
        return np.asarray(a, dtype=np.float16).astype(np.float32)
    if dtype == "fp32":
        return np.array(a, dtype=np.float32, copy=True)
    raise ValueError(dtype)


def to_bf16_bits(v):
    """fp32 -> bf16 raw bits, round to nearest even (finite inputs)."""
    u = np.asarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return (r & np.uint64(0xFFFF)).astype(np.uint16)


def to_fp16(v):
    """fp32 -> fp16, round to nearest even with subnormals (numpy's cast)."""
    with np.errstate(over="ignore"):
        return np.asarray(v, dtype=np.float32).astype(np.float16)


def narrow(v, dtype):
    """fp32 -> storage array of ``dtype`` (bf16 as raw uint16 bits)."""
    if dtype == "fp32":
        return np.asarray(v, dtype=np.float32).copy()
    if dtype == "fp16":
        return to_fp16(v)
    if dtype == "bf16":
        return to_bf16_bits(v)
    raise ValueError(dtype)


def raw_bits(a):
    """Raw bit pattern view used for bit-exact comparisons."""
    a = np.asarray(a)
    if a.dtype == np.float32:
        return a.view(np.uint32)
    if a.dtype == np.float16:
        return a.view(np.uint16)
    return a


def f32_exact_int(a):
    """Finite fp32 values as exact integers times 2^-149: (sign, magnitude).

    IEEE binary32: biased exponent e, fraction f; normal (e > 0) values are
    (2^23 + f) * 2^(e - 150), subnormal (e = 0) values f * 2^-149."""
    bits = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).ravel()
    e = ((bits >> 23) & 0xFF).astype(np.int64)
    f = (bits & 0x7FFFFF).astype(np.int64)
    m = np.where(e > 0, f | 0x800000, f)
    shift = np.maximum(e, 1) - 1
    neg = (bits >> 31).astype(bool)
    return neg, m, shift


def exact_sum_f32(a):
    """Exact sum of finite fp32 values, as an integer X with sum = X * 2^-149."""
    neg, m, shift = f32_exact_int(a)
    total = 0
    for s, mm, sh in zip(neg.tolist(), m.tolist(), shift.tolist()):
        total += -(mm << sh) if s else (mm << sh)
    return total


def rn32_rational(num, den):
    """num / den (integers, den > 0) rounded to binary32, to nearest, ties to
    even, with gradual underflow; overflow gives +-inf."""
    if num == 0:
        return np.float32(0.0)
    sign = -1 if num < 0 else 1
    num = abs(num)
    # e = floor(log2(num / den))
    e = num.bit_length() - den.bit_length()
    if (num << max(0, -e)) < (den << max(0, e)):
        e -= 1
    e = max(e, -126)                      # below the normal range: subnormal spacing 2^-149
    # q = num / den / 2^(e - 23), rounded to an integer (24 significant bits)
    sh = 23 - e
    n2, d2 = (num << sh, den) if sh >= 0 else (num, den << -sh)
    q, r = divmod(n2, d2)
    if 2 * r > d2 or (2 * r == d2 and q & 1):
        q += 1
    if q == 1 << 24:                      # rounding carried into the next binade
        q >>= 1
        e += 1
    if e > 127:
        return np.float32(sign * np.inf)
    return np.float32(sign * float(q) * 2.0 ** (e - 23))
