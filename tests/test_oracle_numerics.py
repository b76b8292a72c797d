"""Pins for the oracle's element formats against exact rational rounding."""

import math

import numpy as np
import pytest

from oracle import numerics
from tests import exact


def _edge_values():
    vals = [0.0, -0.0, 1.0, -1.0, 65504.0, 65519.99, 65520.0, 1e-45, -1e-45,
            6.0e-8, 5.96e-8, 2.98e-8, 2.9802322e-08, 3.0e-8, 1.17549435e-38,
            1.1754942e-38, 3.3895314e38, 3.4e38, 1.0 + 2 ** -8, 1.0 + 2 ** -8 + 2 ** -23,
            1.0 + 3 * 2 ** -8, 1.0 + 2 ** -11, 1.0 + 3 * 2 ** -11, 6.1035156e-05, 6.097555e-05]
    return np.array(vals, dtype=np.float32)


def _random_values(n=4000, seed=0):
    rng = np.random.default_rng(seed)
    bits = rng.integers(0, 1 << 32, size=n, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    return v[np.isfinite(v)]


def _bf16_exact(v):
    r = exact.round_to(exact.frac(v), exact.BF16)
    return r


def _bf16_value(bits):
    return float(np.array([np.uint32(bits) << np.uint32(16)], dtype=np.uint32).view(np.float32)[0])


@pytest.mark.parametrize("src", ["edge", "random"])
def test_bf16_rne_matches_exact_rounding(src):
    v = _edge_values() if src == "edge" else _random_values()
    bits = numerics.to_bf16_bits(v)
    for x, b in zip(v, bits):
        want = _bf16_exact(x)
        got = _bf16_value(b)
        if isinstance(want, float) and math.isinf(want):
            assert math.isinf(got) and (got > 0) == (want > 0)
        else:
            assert exact.frac(got) == want, (float(x), hex(int(b)))
        if x == 0:
            assert math.copysign(1.0, got) == math.copysign(1.0, float(x))


@pytest.mark.parametrize("src", ["edge", "random"])
def test_fp16_rne_matches_exact_rounding(src):
    v = _edge_values() if src == "edge" else _random_values(seed=1)
    h = numerics.to_fp16(v)
    for x, y in zip(v, h):
        want = exact.round_to(exact.frac(x), exact.FP16)
        got = float(y)
        if isinstance(want, float) and math.isinf(want):
            assert math.isinf(got) and (got > 0) == (want > 0)
        else:
            assert exact.frac(got) == want, (float(x), float(y))
        if x == 0:
            assert math.copysign(1.0, got) == math.copysign(1.0, float(x))


def test_widen_is_exact():
    bits = np.arange(0, 1 << 16, 7, dtype=np.uint16)
    w = numerics.widen(bits, "bf16")
    back = numerics.to_bf16_bits(w[np.isfinite(w)])
    assert np.array_equal(back, bits[np.isfinite(w)])
    h = bits.view(np.float16)
    wf = numerics.widen(h, "fp16")
    fin = np.isfinite(wf)
    assert np.array_equal(wf[fin].astype(np.float16).view(np.uint16), bits[fin])


def test_host_keeps_subnormals():
    assert np.float32(1e-45) > 0
    assert np.float32(1e-38) / np.float32(4.0) > 0
