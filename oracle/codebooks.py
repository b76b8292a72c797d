"""Codebooks (test infrastructure only).

All values are computed in float64 and rounded once to float32.

``nf_pages_rule(K)``
    The level rule of [QLORA-2] PATCH 001, ``tests/test_kbit_quantization.py``,
    ``create_normal_float_codebook``: 2^K levels at the N(0,1) quantiles of
    the bin midpoints (2i+1)/(2n), divided by the largest magnitude.  It is
    antisymmetric and has no zero for any K.  Used as an extra test codebook.

``nf(K)``
    The NF codebook of the hot path.  The pages name an "asymmetric
    extra-value / zero trick" for NF4 without giving its constants, while the
    codebook must hold an exact 0 with endpoints -1 and +1.  Reading: take the
    pages' midpoint-quantile rule twice -- at n = 2^K - 1 levels (odd, so its
    centre level is exactly 0) for the 2^(K-1) - 1 negative levels, and at
    n = 2^K levels for the 2^(K-1) positive levels -- add 0.0, and scale each
    side on its own so that its outermost level is exactly -1 / +1.

``fp4()``
    FP4 (E2M1) magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6} with both signs, divided
    by 6 in float32 (one rounding of the exact rational).  Index order: the
    eight negatives (-6 .. -0) then the eight positives (+0 .. +6).  The FP4
    format is named by [PR2051] Summary, which prints no table; the values and
    their order are a reading of that name (standard E2M1 magnitudes).

``lloyd_max_normal(L)``
    The L-level minimum-MSE (Lloyd-Max) quantizer of N(0,1), found by the
    classical fixed-point iteration (centroid of each cell, boundaries at
    midpoints) in float64 with closed-form Gaussian cell moments, made exactly
    symmetric, rounded once to float32.  [ORBIT] methodology audit: published
    checkpoints use a converged Lloyd-Max codebook.

``dynamic_map8()``
    A 256-entry signed "dynamic tree" 8-bit map for the nested absmax codes
    ([PR2051] Summary names the General8 scale code; its table is not on the
    pages).  Built here from the published description of dynamic tree
    quantization (Dettmers et al., "8-bit Optimizers via Block-wise
    Quantization", 2021): a sign, a decimal exponent 10^-z coded by z leading
    zero bits, then a linear fraction in (0.1, 1) taken at the midpoints of
    2^(6-z) equal slots; plus 0 and 1.  Pinned against a bit-by-bit decoding
    of the 256 codes in exact rationals (the GPU path reads the map as data).
"""

import math

import numpy as np
from scipy import special

F32 = np.float32


def _midpoint_quantiles(n):
    """N(0,1) quantiles at the bin midpoints (2i+1)/(2n), i = 0..n-1, float64."""
    i = np.arange(n, dtype=np.float64)
    return special.ndtri((2.0 * i + 1.0) / (2.0 * n))


def nf_pages_rule(K):
    """The pages' symmetric NF level rule (no zero level)."""
    n = 1 << K
    z = _midpoint_quantiles(n)
    return (z / np.max(np.abs(z))).astype(np.float32)


def nf(K):
    """NF_K codebook with an exact zero (see module docstring)."""
    if not 2 <= K <= 8:
        raise ValueError("K must be in 2..8")
    n_odd = (1 << K) - 1
    zo = _midpoint_quantiles(n_odd)
    neg = zo[: (n_odd - 1) // 2]           # strictly negative levels
    neg = neg / (-neg[0])                   # outermost -> exactly -1
    n_even = 1 << K
    ze = _midpoint_quantiles(n_even)
    pos = ze[n_even // 2:]                  # strictly positive levels
    pos = pos / pos[-1]                     # outermost -> exactly +1
    vals = np.concatenate([neg, [0.0], pos])
    return vals.astype(np.float32)


def fp4():
    """FP4 (E2M1) codebook scaled to [-1, 1]."""
    mags = [6.0, 4.0, 3.0, 2.0, 1.5, 1.0, 0.5, 0.0]
    num = np.array([-m for m in mags] + mags[::-1], dtype=np.float32)
    num[7] = np.float32(-0.0)
    return (num / np.float32(6.0)).astype(np.float32)


def _cell_moments(lo, hi):
    """P(lo<X<hi) and E[X; lo<X<hi] for X ~ N(0,1), float64, tail-accurate."""
    # probability: use the side of the distribution that avoids cancellation
    if lo >= 0.0:
        p = special.ndtr(-lo) - special.ndtr(-hi)
    else:
        p = special.ndtr(hi) - special.ndtr(lo)
    phi = lambda t: 0.0 if math.isinf(t) else math.exp(-0.5 * t * t) / math.sqrt(2.0 * math.pi)
    m = phi(lo) - phi(hi)
    return p, m


def lloyd_max_normal(L=16, tol=1e-15, max_iter=200000, return_float64=False):
    """Lloyd-Max quantizer levels for N(0,1) (sorted ascending)."""
    if L < 2 or L % 2:
        raise ValueError("L must be even and >= 2")
    c = _midpoint_quantiles(L)
    for _ in range(max_iter):
        b = 0.5 * (c[:-1] + c[1:])
        edges = np.concatenate([[-math.inf], b, [math.inf]])
        new = np.empty_like(c)
        for i in range(L):
            p, m = _cell_moments(edges[i], edges[i + 1])
            new[i] = m / p
        new = 0.5 * (new - new[::-1])       # exact antisymmetry
        delta = np.max(np.abs(new - c))
        c = new
        if delta < tol:
            break
    return c if return_float64 else c.astype(np.float32)


def dynamic_map8():
    """256-entry signed dynamic-tree map, sorted ascending, float32."""
    pos = []
    for z in range(7):                      # decimal exponent 10^-z
        slots = 1 << (6 - z)                # fraction slots at this exponent
        for f in range(slots):
            # 10^-z * (0.1 + 0.9 * (2f+1) / (2*slots)), as one exact rational
            num = 2 * slots + 9 * (2 * f + 1)
            den = 20 * slots * 10 ** z
            pos.append(num / den)           # correctly rounded float64
    pos = np.array(pos, dtype=np.float64)
    vals = np.concatenate([-pos, [0.0], pos, [1.0]])
    vals = np.sort(vals.astype(np.float32))
    return vals
