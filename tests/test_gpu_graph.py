"""The hot path captured into a HIP graph (as the benchmark runs it) gives, on
every replay, exactly what eager launches give.  Outputs are cleared between
replays, with eager work and synchronisations in between."""

import numpy as np
import pytest

import blockwise_bit_codebook_amd as kb
from blockwise_bit_codebook_amd import synth
from oracle import codebooks, kbit, nested
from tests.gpu_util import bits, case, np_bits, to_dev

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager_and_oracle():
    import torch
    B, K = 64, 4
    x = synth.weight(1024, 1024, "bf16", seed=synth.SEED_WEIGHT_SHAPES, extra=synth.TAIL_EXTRA)
    n = x.size
    nb = kb.n_blocks(n, B)
    cb = to_dev(codebooks.nf(K))
    q = codebooks.dynamic_map8()
    qmap = to_dev(q)
    code_np, a2_np, off = synth.nested_state_synthetic(nb, seed=3)
    A = to_dev(x, "bf16")
    code, a2 = to_dev(code_np), to_dev(a2_np)
    packed = torch.empty(kb.n_words(n, K), dtype=torch.int32, device="cuda")
    absmax = torch.empty(nb, dtype=torch.float32, device="cuda")
    out = torch.empty(n, dtype=torch.bfloat16, device="cuda")

    def step():
        kb.quantize_kbit(A, cb, K, B, absmax=absmax, packed=packed)
        kb.dequantize_4bit_nested(packed, cb, code, qmap, a2, off, n, torch.bfloat16, B, out=out)

    case("graph: eager reference")
    step()
    torch.cuda.synchronize()
    ref = (bits(packed), bits(absmax), bits(out))

    # the oracle agrees with the eager run
    from oracle import numerics
    want_w, want_a = kbit.quantize_packed(numerics.widen(x, "bf16"), codebooks.nf(K), K, B)
    assert np.array_equal(ref[0], want_w)
    assert np.array_equal(ref[1], np_bits(want_a))
    idx = kbit.unpack(want_w, K, n)
    assert np.array_equal(ref[2], np_bits(nested.dequantize(idx, code_np, a2_np, off, q, codebooks.nf(K), B,
                                                            "bf16")))

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    scratch = torch.empty_like(packed)
    for r in range(4):
        case(f"graph: replay {r}")
        packed.zero_()
        absmax.zero_()
        out.zero_()
        kb.quantize_kbit(A, cb, K, B, packed=scratch)     # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(packed), ref[0]), r
        assert np.array_equal(bits(absmax), ref[1]), r
        assert np.array_equal(bits(out), ref[2]), r


@pytest.mark.parametrize("dtype,K", [("fp16", 5), ("fp32", 5), ("fp32", 3), ("bf16", 2), ("fp16", 4)])
def test_graph_replays_other_types(dtype, K):
    # quantize + plain dequantize of other input types and K (two-row
    # 16-bit steps, the fp32 wave-row layout, K = 5's plane-4 chains)
    # captured once and replayed; every replay equals the eager run and the
    # oracle
    import torch
    from oracle import numerics
    from tests.test_gpu_dequantize import _tdt
    B = 64
    x = synth.weight(1024, 1024, dtype, seed=synth.SEED_WEIGHT_SHAPES, extra=synth.TAIL_EXTRA)
    n = x.size
    nb = kb.n_blocks(n, B)
    cb = to_dev(codebooks.nf(K))
    A = to_dev(x, dtype)
    packed = torch.empty(kb.n_words(n, K), dtype=torch.int32, device="cuda")
    absmax = torch.empty(nb, dtype=torch.float32, device="cuda")
    out = torch.empty(n, dtype=_tdt(dtype), device="cuda")

    def step():
        kb.quantize_kbit(A, cb, K, B, absmax=absmax, packed=packed)
        kb.dequantize_kbit(packed, cb, absmax, K, n, _tdt(dtype), B, out=out)

    case(f"graph {dtype} K={K}: eager reference")
    step()
    torch.cuda.synchronize()
    ref = (bits(packed), bits(absmax), bits(out))
    want_w, want_a = kbit.quantize_packed(numerics.widen(x, dtype), codebooks.nf(K), K, B)
    assert np.array_equal(ref[0], want_w)
    assert np.array_equal(ref[1], np_bits(want_a))
    assert np.array_equal(ref[2], np_bits(kbit.dequantize_packed(want_w, want_a, codebooks.nf(K), K, n, B, dtype)))

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    scratch = torch.empty_like(packed)
    for r in range(3):
        case(f"graph {dtype} K={K}: replay {r}")
        packed.zero_()
        absmax.zero_()
        out.zero_()
        kb.quantize_kbit(A, cb, K, B, packed=scratch)     # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(packed), ref[0]), r
        assert np.array_equal(bits(absmax), ref[1]), r
        assert np.array_equal(bits(out), ref[2]), r


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("state", ["three_kernels", "quantize_to_nested"])
def test_graph_whole_chain_with_device_offset(dtype, state):
    # quantize -> nested encode -> nested dequantize (offset read on the
    # device) and the fused linear on the same state, captured as one graph
    # with no host read-back; every replay equals the eager run, and the
    # eager run equals the oracle's chain from the input alone.  The state
    # comes from quantize then quantize_nested_absmax, or from
    # quantize_4bit_nested (two kernels).
    import torch
    from oracle import numerics
    from tests.test_gpu_dequantize import _tdt
    B, K = 64, 4
    rows, cols = 512, 1024
    x = synth.weight(rows, cols, dtype, seed=synth.SEED_WEIGHT_SHAPES)
    n = x.size
    nb = kb.n_blocks(n, B)
    cbn = codebooks.nf(K)
    q = codebooks.dynamic_map8()
    cb, qmap = to_dev(cbn), to_dev(q)
    A = to_dev(x, dtype)
    X = to_dev(synth.normal(16 * cols, seed=5, dtype="bf16"), "bf16").view(16, cols)
    packed = torch.empty(kb.n_words(n, K), dtype=torch.int32, device="cuda")
    absmax = torch.empty(nb, dtype=torch.float32, device="cuda")
    code = torch.empty(nb, dtype=torch.uint8, device="cuda")
    a2 = torch.empty(-(-nb // 256), dtype=torch.float32, device="cuda")
    off = torch.empty(1, dtype=torch.float32, device="cuda")
    ws = torch.empty(kb.lib().kbit_nested_workspace_bytes(nb), dtype=torch.uint8, device="cuda")
    qws = torch.empty(kb.lib().kbit_quantize_nested_workspace_bytes(), dtype=torch.uint8, device="cuda")
    out = torch.empty(n, dtype=_tdt(dtype), device="cuda")
    y = torch.empty((16, rows), dtype=torch.bfloat16, device="cuda")

    def chain():
        if state == "quantize_to_nested":
            kb.quantize_4bit_nested(A, cb, qmap, B, absmax=absmax, packed=packed, absmax_code=code, absmax2=a2,
                                    offset=off, workspace=qws)
        else:
            kb.quantize_kbit(A, cb, K, B, absmax=absmax, packed=packed)
            kb.quantize_nested_absmax(absmax, qmap, absmax_code=code, absmax2=a2, offset=off, workspace=ws)
        kb.dequantize_4bit_nested(packed, cb, code, qmap, a2, off, n, _tdt(dtype), B, out=out)
        kb.linear_4bit(X, packed, cb, rows, B, absmax_code=code, qmap2=qmap, absmax2=a2, offset=off, out=y)

    case(f"graph chain {dtype} {state}: eager")
    chain()
    torch.cuda.synchronize()
    ref = [bits(t) for t in (packed, absmax, code, a2, off, out, y)]
    # the by-value offset gives the same outputs
    out_v = kb.dequantize_4bit_nested(packed, cb, code, qmap, a2, float(off.item()), n, _tdt(dtype), B)
    y_v = kb.linear_4bit(X, packed, cb, rows, B, absmax_code=code, qmap2=qmap, absmax2=a2, offset=float(off.item()))
    torch.cuda.synchronize()
    assert np.array_equal(bits(out_v), ref[5]) and np.array_equal(bits(y_v), ref[6])
    # the oracle's chain from the input alone
    ww, wa = kbit.quantize_packed(numerics.widen(x, dtype), cbn, K, B)
    wc, wa2, woff = nested.encode(wa, q)
    assert np.array_equal(ref[0], ww) and np.array_equal(ref[1], np_bits(wa))
    assert np.array_equal(ref[2], wc) and np.array_equal(ref[3], np_bits(wa2))
    assert ref[4][0] == np.float32(woff).view(np.uint32)
    want = nested.dequantize_packed(ww, wc, wa2, woff, q, cbn, n, B, dtype)
    assert np.array_equal(ref[5], np_bits(want))

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        chain()
    torch.cuda.synchronize()
    for r in range(4):
        case(f"graph chain {dtype} {state}: replay {r}")
        for t in (packed, absmax, code, a2, off, out, y):
            t.zero_()
        kb.quantize_kbit(A, cb, K, B)                       # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t, want_bits in zip((packed, absmax, code, a2, off, out, y), ref):
            assert np.array_equal(bits(t), want_bits), r
