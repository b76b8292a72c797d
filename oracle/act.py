"""W4A4-style activation assignment: token norm, sign flip, FWHT, Lloyd-Max.

Test infrastructure only.  Follows [ORBIT] README (the native activation
launch computes token norms, applies RPBH/FWHT and selects the fixed
Lloyd-Max bins; a packed 4-bit variant of the output exists) and the
methodology audit (direction w'/||w'||, divide by max(||w'||, eps) with
activation_eps = 1e-10 when choosing indices, raw norm stored; block
Hadamard of size equal to the largest power-of-two divisor of d).

Per row r of X (bf16, d columns, d a power of two here so the Hadamard block
is the whole row):
  1. x = exact fp32 widening;
  2. S = sum of x_i^2 over a perfect binary tree of contiguous halves, every
     addition rounded to fp32 (the pages fix no order; this is the reading);
     x_i^2 itself is exact for bf16 inputs;
  3. norm = RN(sqrt(S));
  4. u = x with the sign flipped where the shared sign mask has a 1 bit
     (bit t of word w <-> column 32w + t);
  5. unnormalised Sylvester-Hadamard transform in natural order: for
     h = 1, 2, 4, ..., d/2 in that order, every pair (j, j+h) with j & h == 0
     becomes (RN(u_j + u_{j+h}), RN(u_j - u_{j+h}));
  6. z = RN(u / max(norm, 1e-10f));
  7. idx = first-index argmin of |RN(z - c_i)| over the 16 centroids;
  8. pack idx along the flattened rows with the K = 4 bit-plane layout.
Returns (packed words, norms).

Parity: the transform is pinned against a dense float64 Hadamard product
(scipy.linalg.hadamard), its involution property and Parseval; the norm tree
against math.fsum; the assignment against a scalar brute-force search
(``tests/test_oracle_act.py``).
"""

import numpy as np

from . import kbit
from .numerics import widen

ACT_EPS = np.float32(1e-10)


def tree_sum_rows(q):
    """Row sums over a perfect binary tree of contiguous halves (fp32)."""
    q = np.asarray(q, dtype=np.float32)
    while q.shape[1] > 1:
        q = (q[:, 0::2] + q[:, 1::2]).astype(np.float32)
    return q[:, 0]


def fwht_rows(u):
    """Unnormalised natural-order Walsh-Hadamard transform of each row (fp32)."""
    u = np.array(u, dtype=np.float32, copy=True)
    rows, d = u.shape
    h = 1
    while h < d:
        v = u.reshape(rows, d // (2 * h), 2, h)
        a = v[:, :, 0, :]
        b = v[:, :, 1, :]
        u = np.stack([(a + b).astype(np.float32), (a - b).astype(np.float32)], axis=2)
        u = u.reshape(rows, d)
        h *= 2
    return u


def sign_mask_to_bool(sign_words, d):
    w = np.asarray(sign_words, dtype=np.uint32).ravel()
    t = np.arange(d)
    return ((w[t // 32] >> (t % 32).astype(np.uint32)) & 1).astype(bool)


def assign(x_bits, sign_words, codebook16):
    """Config-5 activation path; x_bits is bf16 raw uint16 [rows, d]."""
    xb = np.asarray(x_bits, dtype=np.uint16)
    rows, d = xb.shape
    if d & (d - 1) or d < 32:
        raise ValueError("d must be a power of two >= 32")
    x = widen(xb, "bf16").reshape(rows, d)
    norms = np.sqrt(tree_sum_rows((x * x).astype(np.float32))).astype(np.float32)
    flip = sign_mask_to_bool(sign_words, d)
    u = np.where(flip[None, :], -x, x).astype(np.float32)
    u = fwht_rows(u)
    den = np.maximum(norms, ACT_EPS).astype(np.float32)
    z = (u / den[:, None]).astype(np.float32)
    idx = kbit.nearest_code(z.ravel(), codebook16)
    return kbit.pack(idx, 4), norms
