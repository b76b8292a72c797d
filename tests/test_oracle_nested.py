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
