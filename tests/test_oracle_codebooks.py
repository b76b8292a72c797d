"""Pins for the oracle's codebooks (NF, FP4, Lloyd-Max, dynamic map)."""

import math
import os
import statistics
from fractions import Fraction

import numpy as np
import pytest
from scipy import integrate

from oracle import codebooks
from tests import exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("K", [2, 3, 4, 5])
def test_nf_structure(K):
    c = codebooks.nf(K)
    assert c.dtype == np.float32 and c.size == 1 << K
    assert np.all(np.diff(c) > 0)                    # sorted, distinct
    assert c[0] == np.float32(-1.0) and c[-1] == np.float32(1.0)
    assert np.count_nonzero(c == 0) == 1
    zero = int(np.flatnonzero(c == 0)[0])
    assert zero == (1 << (K - 1)) - 1                # one more positive level
    assert not np.signbit(c[zero])


@pytest.mark.parametrize("K", [2, 3, 4, 5])
def test_nf_positive_half_is_the_pages_rule(K):
    # the positive levels are the pages' midpoint-quantile levels unchanged
    half = 1 << (K - 1)
    assert np.array_equal(codebooks.nf(K)[half:], codebooks.nf_pages_rule(K)[half:])


@pytest.mark.parametrize("K", [2, 3, 4, 5])
def test_nf_quantiles_against_independent_inverse_cdf(K):
    # statistics.NormalDist uses its own inverse CDF (not scipy's ndtri)
    nd = statistics.NormalDist()
    n_odd, n_even = (1 << K) - 1, 1 << K
    neg = [nd.inv_cdf((2 * i + 1) / (2 * n_odd)) for i in range((n_odd - 1) // 2)]
    pos = [nd.inv_cdf((2 * i + 1) / (2 * n_even)) for i in range(n_even // 2, n_even)]
    want = [v / -neg[0] for v in neg] + [0.0] + [v / pos[-1] for v in pos]
    got = codebooks.nf(K).astype(np.float64)
    assert np.allclose(got, want, rtol=0, atol=2 ** -23)


def test_nf4_close_to_the_pages_rule():
    # same closeness bound the pages use when comparing k=4 with legacy NF4
    assert np.max(np.abs(codebooks.nf(4) - codebooks.nf_pages_rule(4))) < 0.15


@pytest.mark.parametrize("K", [2, 3, 4, 5])
def test_pages_rule_properties(K):
    c = codebooks.nf_pages_rule(K)
    assert c.size == 1 << K and np.all(np.diff(c) > 0)
    assert abs(float(np.max(np.abs(c))) - 1.0) <= 1e-6
    assert np.array_equal(c, -c[::-1])
    assert abs(float(c.mean())) < 0.1


def test_fp4_exact_rationals():
    c = codebooks.fp4()
    mags = [Fraction(v) for v in ("6", "4", "3", "2", "3/2", "1", "1/2", "0")]
    want = [-m / 6 for m in mags] + [m / 6 for m in mags[::-1]]
    assert c.size == 16
    for got, w in zip(c, want):
        assert exact.frac(got) == exact.round_to(w, exact.FP32)
    assert np.signbit(c[7]) and not np.signbit(c[8])
    assert c[0] == -1.0 and c[-1] == 1.0
    assert np.all(np.diff(c) >= 0)


def _golden_lloyd():
    levels, mse = None, None
    with open(os.path.join(GOLDEN, "lloyd_max16_normal.txt")) as f:
        for line in f:
            if line.startswith("levels"):
                levels = [float(v) for v in line.split()[1:]]
            elif line.startswith("mse"):
                mse = float(line.split()[1])
    return np.array(levels), mse


def _phi(t):
    return math.exp(-0.5 * t * t) / math.sqrt(2 * math.pi)


def test_lloyd_max16_against_max_1960_table():
    levels, mse = _golden_lloyd()
    c = codebooks.lloyd_max_normal(16)
    assert np.allclose(c[8:], levels, atol=6e-4)
    assert np.array_equal(c, -c[::-1])
    # MSE by numerical integration, independent of the iteration's closed forms
    c64 = c.astype(np.float64)
    edges = [-math.inf] + list(0.5 * (c64[:-1] + c64[1:])) + [math.inf]
    d = 0.0
    for i in range(16):
        v, _ = integrate.quad(lambda t, ci=c64[i]: (t - ci) ** 2 * _phi(t), edges[i], edges[i + 1])
        d += v
    assert abs(d - mse) < 1e-5          # table value has four significant digits


def test_lloyd_max16_is_a_fixed_point():
    c = codebooks.lloyd_max_normal(16, return_float64=True)
    edges = [-math.inf] + list(0.5 * (c[:-1] + c[1:])) + [math.inf]
    for i in range(16):
        m, _ = integrate.quad(lambda t: t * _phi(t), edges[i], edges[i + 1], epsabs=1e-14, epsrel=1e-13)
        p, _ = integrate.quad(_phi, edges[i], edges[i + 1], epsabs=1e-14, epsrel=1e-13)
        assert abs(m / p - c[i]) < 1e-9


def test_dynamic_map_structure():
    q = codebooks.dynamic_map8()
    assert q.dtype == np.float32 and q.size == 256
    assert np.all(np.diff(q) > 0)
    assert q[-1] == 1.0 and np.count_nonzero(q == 0) == 1
    assert q[0] >= -1.0 and q[0] < -0.99
    pos = q[(q > 0) & (q < 1)]
    neg = q[q < 0]
    assert np.array_equal(np.sort(-neg), pos)         # mirror image apart from +1
    for z in range(7):                                  # 2^(6-z) levels per decade
        lo, hi = 10.0 ** (-z - 1), 10.0 ** (-z)
        assert np.count_nonzero((pos > lo) & (pos < hi)) == 1 << (6 - z)


def _decode_dynamic_code(c):
    """Value of one 8-bit dynamic-tree code, read bit by bit.

    Bit 7 is the sign.  Of the other seven bits, the leading zeros count the
    decimal exponent z (value scale 10^-z), the first one bit marks where the
    fraction starts, and the 6 - z bits after it index one of 2^(6-z) equal
    slots of the linear fraction range (0.1, 1); the slot's midpoint is taken.
    Seven zero bits code 0.  Returns an exact Fraction.
    """
    sign = -1 if c & 0x80 else 1
    m = c & 0x7F
    if m == 0:
        return Fraction(0)
    z = 7 - m.bit_length()                  # leading zeros of the 7-bit field
    nbits = 6 - z                           # fraction bits after the marker
    f = m & ((1 << nbits) - 1)
    slot = Fraction(9, 10) / (1 << nbits)
    frac_part = Fraction(1, 10) + slot * f + slot / 2
    return sign * frac_part / Fraction(10) ** z


def test_dynamic_map_matches_bitwise_decoding():
    """Every entry equals a code of the published dynamic-tree layout, decoded
    bit by bit and rounded once to fp32 by exact rational arithmetic; the
    code with sign bit set and zero magnitude (a second zero) stands for +1.
    """
    want = set()
    for c in range(256):
        if c == 0x80:
            want.add(1.0)
            continue
        want.add(exact.f32(_decode_dynamic_code(c)))
    q = codebooks.dynamic_map8()
    assert len(want) == 256
    assert sorted(want) == [float(v) for v in q]
    # hand-derived landmarks: the finest level 10^-6 * 0.55, the coarsest
    # slot midpoint below 1, 0.1 + 0.9 * 63.5 / 64 = 1271/1280
    assert float(q[127]) == 0.0
    assert float(q[128]) == exact.f32(Fraction(55, 10 ** 8))
    assert float(q[254]) == exact.f32(Fraction(1271, 1280))
