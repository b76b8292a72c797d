"""Pins for the oracle's nested (double-quantized) state."""

import numpy as np
import pytest

from oracle import codebooks, kbit, nested
from blockwise_bit_codebook_amd import synth
from tests import exact


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
def test_reduces_to_plain_path(dtype):
    # offset 0 and absmax2 1: s_b = RN(RN(q * 1) + 0) = q, so the nested
    # decode is the plain decode with absmax = qmap2[code]
    q = codebooks.dynamic_map8()
    cb = codebooks.nf(4)
    rng = np.random.default_rng(2)
    nb, B = 700, 64
    code = rng.integers(0, 256, size=nb, dtype=np.uint8)
    idx = rng.integers(0, 16, size=nb * B - 5, dtype=np.uint8)
    a2 = np.ones(-(-nb // 256), np.float32)
    got = nested.dequantize(idx, code, a2, np.float32(0.0), q, cb, B, dtype)
    want = kbit.dequantize(idx, q[code], cb, B, dtype)
    assert np.array_equal(got.view(np.uint8), want.view(np.uint8))


def _find_fma_canary(rng):
    while True:
        qv, a2, off = (np.float32(v) for v in rng.uniform(-1, 1, 3) * np.array([1, 0.05, 0.02]))
        fused = exact.round_to(exact.frac(qv) * exact.frac(a2) + exact.frac(off), exact.FP32)
        sep = exact.round_to(exact.round_to(exact.frac(qv) * exact.frac(a2), exact.FP32) + exact.frac(off), exact.FP32)
        if fused != sep:
            return qv, a2, off, sep


def test_scale_rebuild_is_separately_rounded():
    rng = np.random.default_rng(7)
    for _ in range(20):
        qv, a2, off, sep = _find_fma_canary(rng)
        qmap = np.array([qv], np.float32)
        s = nested.scales(np.array([0], np.uint8), np.array([a2], np.float32), off, qmap)
        assert exact.frac(s[0]) == sep


def test_group_indexing_with_odd_tail_group():
    q = codebooks.dynamic_map8()
    nb = 256 * 3 + 3
    code = np.arange(nb, dtype=np.uint32).astype(np.uint8)
    a2 = np.array([0.5, 0.25, 2.0, 4.0], np.float32)
    s = nested.scales(code, a2, np.float32(0.125), q)
    for b in (0, 255, 256, 511, 512, 767, 768, 770):
        p = exact.round_to(exact.frac(q[code[b]]) * exact.frac(a2[b // 256]), exact.FP32)
        assert exact.frac(s[b]) == exact.round_to(p + exact.frac(np.float32(0.125)), exact.FP32)


@pytest.mark.parametrize("nb", [1, 255, 256, 257, 1027])
def test_encode_round_trip_bound(nb):
    q = codebooks.dynamic_map8()
    a = np.abs(synth.normal(nb, seed=nb, dtype="fp32", sigma=0.05)).astype(np.float32) + np.float32(0.01)
    code, a2, off = nested.encode(a, q)
    assert code.size == nb and a2.size == -(-nb // 256)
    s = nested.scales(code, a2, off, q).astype(np.float64)
    r = a.astype(np.float64) - float(off)
    # the dynamic map's worst local half-gap is below 0.01 of the group absmax
    g = np.arange(nb) // 256
    gap = float(np.max(np.diff(q.astype(np.float64))))
    assert np.all(np.abs(s - float(off) - r) <= gap / 2 * a2[g] + 1e-6)
    assert abs(float(off) - float(np.mean(a.astype(np.float64)))) <= 1e-7 * float(np.max(a))


def test_encode_matches_definition_small():
    q = codebooks.dynamic_map8()
    a = np.array([0.03, 0.05, 0.07, 0.01, 0.02], np.float32)
    code, a2, off = nested.encode(a, q)
    assert exact.frac(off) == exact.round_to(sum(exact.frac(v) for v in a) / 5, exact.FP32)
    r = [exact.round_to(exact.frac(v) - exact.frac(off), exact.FP32) for v in a]
    amax2 = max(abs(v) for v in r)
    assert exact.frac(a2[0]) == amax2
    for b in range(5):
        xn = exact.f32(r[b] / amax2)
        assert int(code[b]) == exact.nearest_first(xn, q)


def _exact_mean(a):
    return exact.round_to(sum(exact.frac(v) for v in a) / len(a), exact.FP32)


def _same(got, want):
    return exact.frac(got) == want if not isinstance(want, float) else float(got) == want


def test_offset_equals_exact_rational_mean_random():
    rng = np.random.default_rng(31)
    for trial in range(300):
        nb = int(rng.integers(1, 40))
        kind = trial % 4
        if kind == 0:      # typical absmax values
            a = np.abs(rng.normal(0, 0.05, nb)).astype(np.float32)
        elif kind == 1:    # mixed magnitudes and signs, with subnormals
            a = (rng.choice([-1, 1], nb) * np.exp2(rng.uniform(-149, 100, nb))).astype(np.float32)
        elif kind == 2:    # near a common value (long runs of equal exponents)
            a = (np.float32(1.5) + rng.integers(-8, 8, nb).astype(np.float32) * np.float32(2.0 ** -23)).astype(np.float32)
        else:              # huge and tiny together
            a = np.concatenate([np.float32([3e38, -3e38, 1e-45]), rng.normal(0, 1, nb).astype(np.float32)])
        assert _same(nested.mean_offset(a), _exact_mean(a)), (trial, a)


def test_offset_cancellation_and_double_rounding():
    # fp32 accumulation loses the small terms; fp64 does for the second case
    a = np.float32([2.0 ** 24, 1, 1, 1])
    assert exact.frac(nested.mean_offset(a)) == exact.round_to(exact.frac(2.0 ** 24 + 3) / 4, exact.FP32)
    a = np.float32([1e30, 1.0, -1e30])
    assert exact.frac(nested.mean_offset(a)) == exact.round_to(exact.frac(1.0) / 3, exact.FP32)
    # [3, 3*2^-24, 3*2^-60]: the mean 1 + 2^-24 + 2^-60 is just above the fp32
    # midpoint 1 + 2^-24 and rounds up once; through fp64 the 2^-60 is lost,
    # the midpoint ties to even and gives 1.0.  Scaled and mirrored variants.
    for scale in (1.0, 2.0 ** -20, 2.0 ** 40):
        for sgn in (1, -1):
            a = (np.float32([3.0, 3 * 2.0 ** -24, 3 * 2.0 ** -60]) * np.float32(scale * sgn)).astype(np.float32)
            want = _exact_mean(a)
            assert want == exact.frac(np.float32(sgn * scale * (1 + 2.0 ** -23)))
            twice = np.float32(float(sum(exact.frac(v) for v in a)) / 3)
            assert exact.frac(twice) != want
            assert exact.frac(nested.mean_offset(a)) == want


def test_offset_special_values():
    assert nested.mean_offset(np.float32([])) == 0
    assert np.isnan(nested.mean_offset(np.float32([1, np.nan, 2])))
    assert np.isnan(nested.mean_offset(np.float32([np.inf, -np.inf])))
    assert nested.mean_offset(np.float32([1, np.inf])) == np.inf
    assert nested.mean_offset(np.float32([1, -np.inf])) == -np.inf
    assert nested.mean_offset(np.float32([0.3] * 7)) == np.float32(0.3)
    assert nested.mean_offset(np.float32([1e-45, 0, 0, 0])) == 0           # 2^-151 rounds to 0
    assert nested.mean_offset(np.float32([3e-45, 0])) == np.float32(1e-45)  # 1.5 * 2^-149 -> 2 * 2^-149
    big = np.full(1 << 20, 0.25, np.float32)
    big[7] = np.float32(2.0 ** -30)
    assert exact.frac(nested.mean_offset(big)) == _exact_mean(big)


def test_encode_matches_definition_two_groups():
    # 300 blocks: a full group of 256 and a tail of 44, checked element by
    # element with exact rationals (offset, r, group absmax, nearest code)
    q = codebooks.dynamic_map8()
    rng = np.random.default_rng(8)
    a = np.abs(rng.normal(0, 0.03, 300)).astype(np.float32)
    a[17] = 0.0
    code, a2, off = nested.encode(a, q)
    assert exact.frac(off) == _exact_mean(a)
    r = [exact.round_to(exact.frac(v) - exact.frac(off), exact.FP32) for v in a]
    for g, (lo, hi) in enumerate(((0, 256), (256, 300))):
        amax2 = max(abs(v) for v in r[lo:hi])
        assert exact.frac(a2[g]) == amax2
        for b in list(range(lo, hi, 7)) + [hi - 1]:
            xn = exact.f32(r[b] / max(amax2, exact.frac(np.float32(1e-8))))
            assert int(code[b]) == exact.nearest_first(xn, q), b
