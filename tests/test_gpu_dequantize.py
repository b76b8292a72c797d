"""GPU parity: blockwise dequantize and nested dequantize vs the oracle (bit-exact)."""

import numpy as np
import pytest

import blockwise_bit_codebook_amd as kb
from blockwise_bit_codebook_amd import synth
from oracle import codebooks, kbit, nested, numerics
from tests.gpu_util import TORCH_DT, assert_bits_equal, bits, case, np_bits, sha, to_dev

pytestmark = pytest.mark.gpu

DTYPES = ["fp32", "fp16", "bf16"]


def _tdt(dtype):
    import torch
    return getattr(torch, TORCH_DT[dtype])


def run_dequant(words, absmax, cb, K, n, B, dtype):
    import torch
    out = kb.dequantize_kbit(to_dev(words), to_dev(cb), to_dev(absmax), K, n, _tdt(dtype), B)
    torch.cuda.synchronize()
    return bits(out)


def check_dequant(idx, absmax, cb, K, B, dtype, what):
    n = idx.size
    case(f"dequantize {what} dtype={dtype} K={K} B={B} n={n}")
    words = kbit.pack(idx, K)
    got = run_dequant(words, absmax, cb, K, n, B, dtype)
    want = kbit.dequantize(idx, absmax, cb, B, dtype)
    assert_bits_equal(got, np_bits(want), f"dequant {what}")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("K", [2, 3, 4, 5])
@pytest.mark.parametrize("B", [32, 64])
def test_small_sizes(dtype, K, B):
    rng = np.random.default_rng(K * 100 + B)
    for n in (1, 7, 31, 32, 33, 63, 64, 65, 511, 512, 513, 1000, 2049, 4097, 65613):
        idx = synth.uniform_indices(n, K, seed=n)
        a = rng.uniform(0, 4, size=kb.n_blocks(n, B)).astype(np.float32)
        check_dequant(idx, a, codebooks.nf(K), K, B, dtype, f"small n={n}")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("B", [32, 64, 128, 256, 512, 1024, 2048, 4096])
def test_block_sizes(dtype, B):
    n = 5 * 4096 + 999
    idx = synth.uniform_indices(n, 4, seed=B)
    a = np.random.default_rng(B).uniform(0, 3, size=kb.n_blocks(n, B)).astype(np.float32)
    check_dequant(idx, a, codebooks.nf(4), 4, B, dtype, "bsweep")


@pytest.mark.parametrize("dtype", DTYPES)
def test_rounding_edge_scales(dtype):
    # scales that push products into fp16/bf16 subnormals, overflow and ties
    n = 64 * 12
    idx = synth.uniform_indices(n, 4, seed=5)
    a = np.array([1e-39, 3e-41, 2.5e-38, 7e4, 1e30, 6.1e-5, 5.9e-8, 0.0, 65504.0, 1.0, 3.4e38, 1e-45],
                 np.float32)
    for cb in (codebooks.nf(4), codebooks.fp4()):
        check_dequant(idx, a, cb, 4, 64, dtype, "edge scales")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_round_trip_configs(dtype):
    # 65,536 fp32 N(0,1) K=4 B=32 round trip, decoding quantize's own output
    import torch
    x = synth.round_trip_fp32()
    cb = codebooks.nf(4)
    packed, absmax = kb.quantize_kbit(to_dev(x), to_dev(cb), 4, 32)
    out = kb.dequantize_kbit(packed, to_dev(cb), absmax, 4, x.size, _tdt(dtype), 32)
    torch.cuda.synchronize()
    idx, a = kbit.quantize(x, cb, 32)
    assert_bits_equal(bits(out), np_bits(kbit.dequantize(idx, a, cb, 32, dtype)), "round trip")


@pytest.mark.parametrize("K", [2, 3, 4, 5])
def test_k_sweep_bf16_decode(K):
    # 2^24 + 17 elements; decode to bf16 and fp32
    n = (1 << 24) + 17
    idx = synth.uniform_indices(n, K, seed=K)
    a = np.abs(synth.normal(kb.n_blocks(n, 32), seed=K, dtype="fp32")) + np.float32(0.5)
    words = kbit.pack(idx, K)
    for dtype in ("bf16", "fp32"):
        case(f"dequant k sweep K={K} {dtype}")
        got = run_dequant(words, a, codebooks.nf(K), K, n, 32, dtype)
        assert_bits_equal(got, np_bits(kbit.dequantize(idx, a, codebooks.nf(K), 32, dtype)), "k sweep")


# --------------------------------------------------------------------------
# nested
# --------------------------------------------------------------------------
def run_nested(words, code, a2, off, q, cb, n, B, dtype):
    import torch
    out = kb.dequantize_4bit_nested(to_dev(words), to_dev(cb), to_dev(code), to_dev(q), to_dev(a2), off, n,
                                    _tdt(dtype), B)
    torch.cuda.synchronize()
    return bits(out)


def check_nested(idx, code, a2, off, q, cb, B, dtype, what):
    n = idx.size
    case(f"nested {what} dtype={dtype} B={B} n={n}")
    got = run_nested(kbit.pack(idx, 4), code, a2, off, q, cb, n, B, dtype)
    want = nested.dequantize(idx, code, a2, off, q, cb, B, dtype)
    assert_bits_equal(got, np_bits(want), f"nested {what}")


def _weight_state(rows, cols, extra, dtype, cbname, B, seed):
    """Nested state of a N(0,0.02) weight's real block absmax, plus uniform
    random 4-bit indices (the decode does not depend on where they came from)."""
    x = numerics.widen(synth.weight(rows, cols, dtype, seed, extra=extra), dtype)
    cb = codebooks.nf(4) if cbname == "nf4" else codebooks.fp4()
    a = kbit.block_absmax(x, B)
    q = codebooks.dynamic_map8()
    code, a2, off = nested.encode(a, q)
    idx = synth.uniform_indices(x.size, 4, seed=seed + B)
    return idx, code, a2, off, q, cb


@pytest.mark.parametrize("cbname", ["nf4", "fp4"])
@pytest.mark.parametrize("dtype", DTYPES)
def test_nested_square4096_cells(cbname, dtype):
    idx, code, a2, off, q, cb = _weight_state(4096, 4096, 0, dtype, cbname, 64, synth.SEED_WEIGHT_SQUARE)
    check_nested(idx, code, a2, off, q, cb, 64, dtype, f"4096^2 {cbname}")


@pytest.mark.parametrize("shape", ["wide11008", "tall11008"])
@pytest.mark.parametrize("cbname", ["nf4", "fp4"])
def test_nested_llama_shapes_with_tail_group(shape, cbname):
    r, c = synth.WEIGHT_SHAPES[shape]
    for dtype in DTYPES:
        idx, code, a2, off, q, cb = _weight_state(r, c, synth.TAIL_EXTRA, dtype, cbname, 64,
                                                  synth.SEED_WEIGHT_SHAPES)
        assert code.size % 256 == 3                      # odd tail group of 3 blocks
        check_nested(idx, code, a2, off, q, cb, 64, dtype, f"{shape} {cbname}")


@pytest.mark.parametrize("B", [32, 64, 128, 256, 512, 1024, 2048, 4096])
def test_nested_block_sizes(B):
    for dtype in DTYPES:
        idx, code, a2, off, q, cb = _weight_state(4096, 4096, synth.TAIL_EXTRA, dtype, "nf4", B, 11)
        check_nested(idx, code, a2, off, q, cb, B, dtype, "bsweep")


def _canary_map(a2, off, rng):
    """256 sorted map values q for which RN(q*a2 + off) (fused) differs from
    RN(RN(q*a2) + off) (separately rounded), checked with exact rationals."""
    from tests import exact
    out = set()
    while len(out) < 256:
        qv = np.float32(rng.uniform(-1, 1))
        fused = exact.round_to(exact.frac(qv) * exact.frac(a2) + exact.frac(off), exact.FP32)
        sep = exact.round_to(exact.round_to(exact.frac(qv) * exact.frac(a2), exact.FP32) + exact.frac(off),
                             exact.FP32)
        if fused != sep:
            out.add(float(qv))
    return np.sort(np.array(sorted(out), np.float32))


def test_nested_fma_canary():
    # every scale is a case where a fused multiply-add would round differently
    rng = np.random.default_rng(11)
    a2v, offv = np.float32(0.0371), np.float32(0.01237)
    q = _canary_map(a2v, offv, rng)
    B, nb = 32, 256
    code = np.arange(nb, dtype=np.uint32).astype(np.uint8)
    idx = synth.uniform_indices(nb * B, 4, seed=3)
    for dtype in DTYPES:
        check_nested(idx, code, np.array([a2v], np.float32), offv, q, codebooks.nf(4), B, dtype, "fma canary")


def test_nested_reduces_to_plain():
    import torch
    n, B = 64 * 1000 + 13, 64
    idx = synth.uniform_indices(n, 4, seed=9)
    q = codebooks.dynamic_map8()
    code = synth.uniform_indices(kb.n_blocks(n, B), 8, seed=10)
    a2 = np.ones(kb.n_blocks(kb.n_blocks(n, B), 256), np.float32)
    words = kbit.pack(idx, 4)
    got = run_nested(words, code, a2, np.float32(0.0), q, codebooks.nf(4), n, B, "bf16")
    plain = run_dequant(words, q[code], codebooks.nf(4), 4, n, B, "bf16")
    assert_bits_equal(got, plain, "nested == plain")


def test_nested_full_8192_square():
    # the measured workload (8192 x 8192 + 192, blocksize 64, groups of 256), 6 cells
    n = 8192 * 8192 + synth.TAIL_EXTRA
    idx = synth.uniform_indices(n, 4, seed=21)
    words = kbit.pack(idx, 4)
    x = synth.weight(8192, 8192, "fp32", 11, extra=synth.TAIL_EXTRA)
    q = codebooks.dynamic_map8()
    code, a2, off = nested.encode(kbit.block_absmax(x, 64), q)
    del x
    for cbname in ("nf4", "fp4"):
        cb = codebooks.nf(4) if cbname == "nf4" else codebooks.fp4()
        for dtype in DTYPES:
            case(f"nested 8192^2 {cbname} {dtype}")
            got = run_nested(words, code, a2, off, q, cb, n, 64, dtype)
            want = nested.dequantize(idx, code, a2, off, q, cb, 64, dtype)
            assert_bits_equal(got, np_bits(want), f"nested 8192^2 {cbname} {dtype}")


def test_nested_input_immutability_and_determinism():
    import torch
    n, B = 1 << 20, 64
    idx = synth.uniform_indices(n, 4, seed=1)
    q = codebooks.dynamic_map8()
    code = synth.uniform_indices(n // B, 8, seed=2)
    a2 = np.full(n // B // 256, 0.03, np.float32)
    ins = [to_dev(kbit.pack(idx, 4)), to_dev(codebooks.nf(4)), to_dev(code), to_dev(q), to_dev(a2)]
    h = [sha(t) for t in ins]
    o1 = kb.dequantize_4bit_nested(*ins, 0.01, n, torch.bfloat16, B)
    o2 = kb.dequantize_4bit_nested(*ins, 0.01, n, torch.bfloat16, B)
    torch.cuda.synchronize()
    assert [sha(t) for t in ins] == h
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
