"""W4A4-style activation assignment: token norm, sign flip, FWHT, Lloyd-Max.

Test infrastructure only.  Follows [ORBIT] README (the native activation
launch computes token norms, applies RPBH/FWHT and selects the fixed
Lloyd-Max bins; a packed 4-bit variant of the output exists), the
methodology audit (direction w'/||w'||, divide by max(||w'||, eps) with
activation_eps = 1e-10 when choosing indices, raw norm stored; block
Hadamard of size h equal to the largest power-of-two divisor of d, so
d = 3840 and d = 8960 give h = 256) and the native-kernels CARD.md (a
blocked case with d = 12288 and h = 4096 is among the tested ones).

Per row r of X (bf16, d columns, d a multiple of 32; h = largest power of
two dividing d; the row is d/h blocks of h contiguous columns):
  1. x = exact fp32 widening;
  2. S = sum of x_i^2: within each block over a perfect binary tree of
     contiguous halves, then the block sums added left to right, every
     addition rounded to fp32 (the pages fix no order; this is the
     reading, and for d = h it is the plain tree); x_i^2 is exact for bf16;
  3. norm = RN(sqrt(S));
  4. u_i = x_{perm[i]} (identity when no permutation is given: the pages do
     not say how the permutation of RPBH is drawn, so it is an input), then
     the sign of u_i flipped where the shared sign mask has a 1 bit (bit t
     of word w <-> column 32w + t);
  5. unnormalised Sylvester-Hadamard transform of every block in natural
     order: for s = 1, 2, 4, ..., h/2 in that order, every pair (j, j+s)
     with j & s == 0 becomes (RN(u_j + u_{j+s}), RN(u_j - u_{j+s}));
     pairs never leave a block because s < h and blocks start at multiples
     of h;
  6. z = RN(u / max(norm, 1e-10f)), the max keeping a NaN norm NaN (as
     numpy's and torch's maximum do), so every z of such a row is NaN;
  7. idx = first-index argmin of |RN(z - c_i)| over the 16 centroids;
  8. pack idx along the flattened rows with the K = 4 bit-plane layout.
Returns (packed words, norms).

Parity: the transform is pinned against a dense float64 block-diagonal
Hadamard product (scipy.linalg.hadamard), its involution property and
Parseval; the block size against the audit's examples; the norm against
math.fsum and constructed rounding cases; the assignment against a scalar
brute-force search (``tests/test_oracle_act.py``).
"""

import numpy as np

from . import kbit
from .numerics import widen

ACT_EPS = np.float32(1e-10)


def hadamard_block(d):
    """Block size of the block Hadamard for row length d: the largest power
    of two dividing d (methodology audit)."""
    d = int(d)
    if d <= 0:
        raise ValueError("d must be positive")
    return d & -d


def tree_sum_rows(q):
    """Row sums over a perfect binary tree of contiguous halves (fp32)."""
    q = np.asarray(q, dtype=np.float32)
    while q.shape[1] > 1:
        q = (q[:, 0::2] + q[:, 1::2]).astype(np.float32)
    return q[:, 0]


def token_sum_rows(q, h):
    """Per-block tree sums of each row, then added block after block (fp32)."""
    q = np.asarray(q, dtype=np.float32)
    rows, d = q.shape
    nblk = d // h
    blocks = tree_sum_rows(q.reshape(rows * nblk, h)).reshape(rows, nblk)
    s = blocks[:, 0].copy()
    for b in range(1, nblk):
        s = (s + blocks[:, b]).astype(np.float32)
    return s


def fwht_rows(u, h=None):
    """Unnormalised natural-order Walsh-Hadamard transform of every block of
    h contiguous columns of each row (fp32); h defaults to the row length."""
    u = np.array(u, dtype=np.float32, copy=True)
    rows, d = u.shape
    if h is None:
        h = d
    if h & (h - 1) or d % h:
        raise ValueError("h must be a power of two dividing d")
    s = 1
    while s < h:
        v = u.reshape(rows, d // (2 * s), 2, s)
        a = v[:, :, 0, :]
        b = v[:, :, 1, :]
        u = np.stack([(a + b).astype(np.float32), (a - b).astype(np.float32)], axis=2)
        u = u.reshape(rows, d)
        s *= 2
    return u


def sign_mask_to_bool(sign_words, d):
    w = np.asarray(sign_words, dtype=np.uint32).ravel()
    t = np.arange(d)
    return ((w[t // 32] >> (t % 32).astype(np.uint32)) & 1).astype(bool)


def assign(x_bits, sign_words, codebook16, perm=None):
    """Config-5 activation path; x_bits is bf16 raw uint16 [rows, d].

    perm: optional length-d permutation (u_i = x_{perm[i]} before the sign
    flip)."""
    xb = np.asarray(x_bits, dtype=np.uint16)
    rows, d = xb.shape
    if d < 32 or d % 32:
        raise ValueError("d must be a positive multiple of 32")
    h = hadamard_block(d)
    x = widen(xb, "bf16").reshape(rows, d)
    norms = np.sqrt(token_sum_rows((x * x).astype(np.float32), h)).astype(np.float32)
    if perm is not None:
        p = np.asarray(perm, dtype=np.int64).ravel()
        if p.shape != (d,) or not np.array_equal(np.sort(p), np.arange(d)):
            raise ValueError("perm must be a permutation of 0..d-1")
        x = x[:, p]
    flip = sign_mask_to_bool(sign_words, d)
    u = np.where(flip[None, :], -x, x).astype(np.float32)
    u = fwht_rows(u, h)
    den = np.maximum(norms, ACT_EPS).astype(np.float32)
    z = (u / den[:, None]).astype(np.float32)
    idx = kbit.nearest_code(z.ravel(), codebook16)
    return kbit.pack(idx, 4), norms
