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


def test_other_maps():
    a = np.abs(synth.normal(3000, seed=4, dtype="fp32", sigma=0.05)).astype(np.float32)
    q = codebooks.dynamic_map8()
    check(a, q[::-1].copy(), "unsorted map")
    qd = q.copy()
    qd[100:110] = qd[100]
    check(a, qd, "duplicates")
    check(a, np.linspace(-1, 1, 256).astype(np.float32), "linear map")


def test_chain_quantize_encode_nested_dequantize():
    # 8192 x 8192 bf16 weight, B = 64: quantize, encode the absmax on the GPU,
    # nested-dequantize; state in full, outputs sampled
    import torch
    rows = cols = 8192
    B = 64
    x = synth.weight(rows, cols, "bf16", seed=synth.SEED_WEIGHT_SHAPES)
    cb = codebooks.nf(4)
    q = codebooks.dynamic_map8()
    case("nested chain 8192x8192 bf16")
    A = to_dev(x, "bf16")
    packed, absmax = kb.quantize_kbit(A, to_dev(cb), 4, B)
    code, a2, off = kb.quantize_nested_absmax(absmax, to_dev(q))
    torch.cuda.synchronize()
    wc, wa2, woff = nested.encode(bits(absmax).view(np.float32), q)
    assert bits(off)[0] == np.float32(woff).view(np.uint32)
    assert_bits_equal(bits(a2), np_bits(wa2), "absmax2")
    assert_bits_equal(bits(code), wc, "codes")
    out = kb.dequantize_4bit_nested(packed, to_dev(cb), code, to_dev(q), a2, float(off.item()), x.size,
                                    torch.bfloat16, B)
    torch.cuda.synchronize()
    got = bits(out)
    words = bits(packed)
    rng = np.random.default_rng(1)
    for r in np.concatenate([[0, rows - 1], rng.integers(0, rows, 20)]):
        lo, hi = int(r) * cols, (int(r) + 1) * cols
        blo, bhi = lo // B, hi // B
        idx = kbit.unpack(words[lo // 32 * 4:hi // 32 * 4], 4, cols)
        s = nested.scales(wc, wa2, woff, q)[blo:bhi]
        want = numerics.narrow(kbit.dequantize_values(idx, s, cb, B), "bf16")
        assert_bits_equal(got[lo:hi], want, f"out row {r}")
