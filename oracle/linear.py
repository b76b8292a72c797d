"""Linear layer over 4-bit quantized weights (reference for the fused kernel).

Test infrastructure only.  [PR2051] Summary names the consumer: a
dequantize-plus-linear path, out = X @ W^T with W decoded from the 4-bit
state.  Reading used here (the pages do not fix the product's summation
order):

* W is exactly the bf16 output of the plain or nested dequantize of the
  state (``kbit.dequantize_packed`` / ``nested.dequantize_packed``),
  reshaped to [N, K];
* the reference value is the sum of the exact products X[m][k] * W[n][k],
  computed in float64 (each bf16 x bf16 product is exact there; the float64
  sum of K terms differs from the exact sum by at most K * 2^-53 * sum|p|);
* a kernel that adds the K exact products in fp32, in any order or tree,
  makes at most K - 1 additions on the path of any one product, so it is
  within gamma(K - 1) * sum_k |X[m][k] * W[n][k]| of the exact sum, with
  gamma(j) = j*u / (1 - j*u) (the classic bound for floating-point
  summation).  The unit u is 2^-23, the error of one fp32 addition under
  any faithful rounding (round to nearest would give 2^-24): the rounding
  inside a matrix-core accumulation is not documented, so the bound
  assumes only that each addition's result is one of the two fp32 values
  around the exact one.  Rounding the result to bf16 adds at most 2^-8 of
  the value.

Parity: pinned in ``tests/test_oracle_linear.py`` (reference against exact
rational sums; the bound against its derivation on worst-case inputs).
"""

import numpy as np

from . import kbit, nested
from .numerics import widen


def weights_bf16(words, codebook16, N, K, B, absmax=None, code=None, qmap2=None, absmax2=None, offset=None):
    """Decoded bf16 weight bits [N, K] (plain fp32 absmax or the nested state)."""
    n = N * K
    if code is None:
        w = kbit.dequantize_packed(words, absmax, codebook16, 4, n, B, "bf16")
    else:
        w = nested.dequantize_packed(words, code, absmax2, offset, qmap2, codebook16, n, B, "bf16")
    return np.asarray(w, dtype=np.uint16).reshape(N, K)


def reference(x_bits, w_bits):
    """(sum of exact products in float64 [M, N], sum of |products| [M, N])."""
    x = widen(np.asarray(x_bits, np.uint16), "bf16").astype(np.float64)
    w = widen(np.asarray(w_bits, np.uint16), "bf16").astype(np.float64)
    return x @ w.T, np.abs(x) @ np.abs(w).T


def tolerance(abs_sum, K):
    """Largest distance of an fp32 sum of K terms (any order or tree,
    faithful rounding) from the exact sum, before the output rounding."""
    j = (K - 1) * 2.0 ** -23
    return j / (1.0 - j) * abs_sum
