"""GPU parity: nested-state encoder (mean offset, group absmax, 8-bit codes).

Bar: bit-exact against ``oracle.nested.encode`` on the same inputs.
"""

import numpy as np
import pytest

import blockwise_bit_codebook_amd as kb
from blockwise_bit_codebook_amd import synth
from oracle import codebooks, kbit, nested, numerics
from tests.gpu_util import assert_bits_equal, bits, case, np_bits, to_dev

pytestmark = pytest.mark.gpu


def run_encode(a, q):
    import torch
    code, a2, off = kb.quantize_nested_absmax(to_dev(np.ascontiguousarray(a, np.float32)), to_dev(q))
    torch.cuda.synchronize()
    return bits(code), bits(a2), bits(off)[0]


def check(a, q, what):
    a = np.ascontiguousarray(a, np.float32)
    case(f"nested encode {what} nb={a.size}")
    code, a2, off = run_encode(a, q)
    wc, wa2, woff = nested.encode(a, q)
    assert off == np.float32(woff).view(np.uint32), (what, hex(off), hex(np.float32(woff).view(np.uint32)))
    assert_bits_equal(a2, np_bits(wa2), f"absmax2 {what}")
    assert_bits_equal(code, wc, f"codes {what}")


@pytest.mark.parametrize("nb", [1, 2, 7, 255, 256, 257, 1000, 4099, 65537])
def test_sizes(nb):
    a = np.abs(synth.normal(nb, seed=nb, dtype="fp32", sigma=0.05)).astype(np.float32)
    check(a, codebooks.dynamic_map8(), "sizes")


def test_many_workgroups():
    # more blocks than 256 workgroups x 4096: every workgroup loops
    nb = 256 * 4096 * 3 + 17
    a = np.abs(synth.normal(nb, seed=3, dtype="fp32", sigma=0.03)).astype(np.float32)
    check(a, codebooks.dynamic_map8(), "many groups")


def test_special_values():
    q = codebooks.dynamic_map8()
    base = np.abs(synth.normal(700, seed=9, dtype="fp32", sigma=0.05)).astype(np.float32)
    for name, patch in [("nan", {5: np.nan}), ("posinf", {300: np.inf}), ("neginf", {3: -np.inf}),
                        ("both inf", {1: np.inf, 600: -np.inf}), ("negatives", {k: -0.3 for k in range(0, 700, 9)}),
                        ("subnormal", {k: 1e-42 for k in range(0, 700, 5)}), ("huge", {10: 3e38, 20: 3e38, 30: -1e38})]:
        a = base.copy()
        for k, v in patch.items():
            a[k] = v
        check(a, q, name)
    check(np.zeros(513, np.float32), q, "zeros")
    check(np.full(300, 1e-45, np.float32), q, "all tiny")
    check(np.float32([3.0, 3 * 2.0 ** -24, 3 * 2.0 ** -60]), q, "single rounding")


def test_wide_exponent_spread():
    # magnitudes from the subnormals up to 2^100 with mixed signs: every wave
    # of the significand sums has values inside and far below its top 24
    # binades, and the positive and negative totals nearly cancel
    rng = np.random.default_rng(31)
    nb = 70001
    e = rng.integers(-149, 100, nb)
    sign = np.where(rng.random(nb) < 0.5, -1.0, 1.0)
    a = (sign * np.ldexp(1.0 + rng.random(nb), e)).astype(np.float32)
    check(a, codebooks.dynamic_map8(), "wide spread")
    a[np.argmax(np.abs(a))] = 0.0
    check(a, codebooks.dynamic_map8(), "wide spread, top removed")


def test_other_maps():
    a = np.abs(synth.normal(3000, seed=4, dtype="fp32", sigma=0.05)).astype(np.float32)
    q = codebooks.dynamic_map8()
    check(a, q[::-1].copy(), "unsorted map")
    qd = q.copy()
    qd[100:110] = qd[100]
    check(a, qd, "duplicates")
    check(a, np.linspace(-1, 1, 256).astype(np.float32), "linear map")


def _bucket_edge_values():
    # floats on and next to the starts of the code search's key buckets
    # (keys of [-1, 1] in steps of 2^18 of the order key), both signs
    k = np.arange(0, 0x3F800000, 1 << 18, dtype=np.int64)[::80]
    bits = np.concatenate([k, k + 1, np.maximum(k - 1, 0)]).astype(np.uint32)
    pos = bits.view(np.float32)
    return np.concatenate([pos, -pos]).astype(np.float32)


@pytest.mark.parametrize("name", ["dense", "wide", "signed zeros", "tiny", "edges"])
def test_sorted_maps_for_the_bucket_table(name):
    # sorted maps that stress the search's bucket table: many entries in one
    # bucket (the walk), entries outside [-1, 1] (counted everywhere or
    # nowhere), -0 before +0, subnormal entries, map entries on bucket edges
    rng = np.random.default_rng(77)
    q = codebooks.dynamic_map8()
    if name == "dense":
        q = np.sort(np.float32(0.3) + np.float32(2.0 ** -20) * np.arange(256, dtype=np.float32)).astype(np.float32)
    elif name == "wide":
        q = np.linspace(-4, 4, 256).astype(np.float32)
    elif name == "signed zeros":
        q = np.sort(rng.uniform(-1, 1, 256)).astype(np.float32)
        q[127], q[128] = np.float32(-0.0), np.float32(0.0)
    elif name == "tiny":
        q = np.sort(np.concatenate([rng.uniform(-1, 1, 200), np.float32(1e-42) * np.arange(-28, 28)])).astype(np.float32)
    else:
        e = _bucket_edge_values()
        q = np.sort(rng.choice(e, 256, replace=False)).astype(np.float32)
    # signed values around a mean, so that r / absmax2 spans [-1, 1]
    a = synth.normal(5000, seed=78, dtype="fp32", sigma=0.05).astype(np.float32)
    a[:64] = np.float32(a.mean())
    check(a, q, f"bucket table, {name} map")


@pytest.mark.parametrize("shape", ["wide11008", "tall11008", "square8192"])
def test_chain_quantize_encode_nested_dequantize(shape):
    # bf16 weight of each shape plus a 192-element tail, B = 64: quantize,
    # encode the absmax and nested-dequantize on the GPU as one stream-ordered
    # chain; the oracle runs the same chain from the input alone, and every
    # stage is compared in full
    import torch
    rows, cols = synth.WEIGHT_SHAPES[shape]
    B = 64
    x = synth.weight(rows, cols, "bf16", seed=synth.SEED_WEIGHT_SHAPES, extra=synth.TAIL_EXTRA)
    n = x.size
    cb = codebooks.nf(4)
    q = codebooks.dynamic_map8()
    case(f"nested chain {shape}+{synth.TAIL_EXTRA} bf16")
    packed, absmax = kb.quantize_kbit(to_dev(x, "bf16"), to_dev(cb), 4, B)
    code, a2, off = kb.quantize_nested_absmax(absmax, to_dev(q))
    # the offset stays on the device: the kernel reads it (no host round trip)
    out = kb.dequantize_4bit_nested(packed, to_dev(cb), code, to_dev(q), a2, off, n, torch.bfloat16, B)
    torch.cuda.synchronize()
    ww, wa = kbit.quantize_packed(numerics.widen(x, "bf16"), cb, 4, B)
    assert_bits_equal(bits(absmax), np_bits(wa), "absmax")
    assert_bits_equal(bits(packed), ww, "words")
    wc, wa2, woff = nested.encode(wa, q)
    assert bits(off)[0] == np.float32(woff).view(np.uint32)
    assert_bits_equal(bits(a2), np_bits(wa2), "absmax2")
    assert_bits_equal(bits(code), wc, "codes")
    want = nested.dequantize_packed(ww, wc, wa2, woff, q, cb, n, B, "bf16")
    assert_bits_equal(bits(out), np_bits(want), "out")
