"""GPU parity over seeded random configurations: input type, K, blocksize,
ragged length, magnitude and codebook kind (NF, random sorted, sorted with a
repeated entry, unsorted) drawn per seed.  Quantize (words and absmax) and
the dequantize of the kernel's own words are compared bit for bit with the
oracle, with fp32 and with E4M4 block scales; the nested chain (quantize,
nested-state encode, fused nested dequantize), quantize straight to the
nested state (quantize_4bit_nested) and the activation
assignment (random width, rows, codebook scale, permutation) likewise; the
fused 4-bit linear (random M, N, K, blocksize) within its fp32-sum bound."""

import numpy as np
import pytest

import blockwise_bit_codebook_amd as kb
from blockwise_bit_codebook_amd import synth
from oracle import codebooks, e4m4, kbit, numerics
from tests.gpu_util import assert_bits_equal, bits, case, np_bits, to_dev
from tests.test_gpu_dequantize import _tdt

pytestmark = pytest.mark.gpu


def _codebook(rng, kind, K):
    C = 1 << K
    if kind == "nf":
        return codebooks.nf(K)
    c = np.sort(rng.uniform(-1.0, 1.0, C)).astype(np.float32)
    if kind == "sorted":
        return c
    if kind == "repeat":                       # two equal neighbours
        j = int(rng.integers(1, C))
        c[j] = c[j - 1]
        return c
    return rng.permutation(c).astype(np.float32)  # unsorted: the exact path


def _config(seed):
    rng = np.random.default_rng(seed)
    dtype = ["fp32", "fp16", "bf16"][int(rng.integers(3))]
    K = int(rng.integers(2, 6))
    B = 1 << int(rng.integers(5, 13))
    n = int(rng.integers(1, 300_000))
    kind = ["nf", "nf", "sorted", "repeat", "unsorted"][int(rng.integers(5))]
    sigma = float(10.0 ** rng.uniform(-3, 1))
    return rng, dtype, K, B, n, kind, sigma


@pytest.mark.parametrize("seed", range(96))
def test_random_config(seed):
    import torch
    rng, dtype, K, B, n, kind, sigma = _config(seed)
    cb = _codebook(rng, kind, K)
    x = synth.normal(n, seed=9000 + seed, dtype=dtype, sigma=sigma)
    case(f"random config seed={seed} dtype={dtype} K={K} B={B} n={n} codebook={kind} sigma={sigma:.3g}")
    packed, absmax = kb.quantize_kbit(to_dev(x, dtype), to_dev(cb), K, B)
    torch.cuda.synchronize()
    words, am = bits(packed), bits(absmax)
    want_w, want_a = kbit.quantize_packed(numerics.widen(x, dtype), cb, K, B)
    assert_bits_equal(am, np_bits(want_a), "absmax")
    assert_bits_equal(words, want_w, "words")
    out = kb.dequantize_kbit(packed, to_dev(cb), absmax, K, n, _tdt(dtype), B)
    torch.cuda.synchronize()
    want = kbit.dequantize_packed(want_w, want_a, cb, K, n, B, dtype)
    assert_bits_equal(bits(out), np_bits(want), "dequantize")


@pytest.mark.parametrize("seed", range(1000, 1048))
def test_random_config_e4m4_scales(seed):
    import torch
    rng, dtype, K, B, n, kind, sigma = _config(seed)
    cb = _codebook(rng, kind, K)
    x = synth.normal(n, seed=9000 + seed, dtype=dtype, sigma=sigma)
    case(f"random config e4m4 seed={seed} dtype={dtype} K={K} B={B} n={n} codebook={kind} sigma={sigma:.3g}")
    packed, code = kb.quantize_kbit(to_dev(x, dtype), to_dev(cb), K, B, absmax_format="e4m4")
    torch.cuda.synchronize()
    want_w, want_c = e4m4.quantize_packed(numerics.widen(x, dtype), cb, K, B)
    assert_bits_equal(bits(code), want_c, "e4m4 codes")
    assert_bits_equal(bits(packed), want_w, "words")
    out = kb.dequantize_kbit(packed, to_dev(cb), code, K, n, _tdt(dtype), B)
    torch.cuda.synchronize()
    want = e4m4.dequantize(kbit.unpack(want_w, K, n), want_c, cb, B, dtype)
    assert_bits_equal(bits(out), np_bits(want), "dequantize")


@pytest.mark.parametrize("seed", range(2000, 2032))
def test_random_config_nested(seed):
    # quantize (K = 4) -> nested state of the block absmax -> fused nested
    # dequantize, all on the GPU; every stage against the oracle
    import torch
    from oracle import nested
    rng, dtype, _, B, n, kind, sigma = _config(seed)
    cb = codebooks.nf(4) if kind in ("nf", "unsorted") else _codebook(rng, "sorted", 4)
    q = codebooks.dynamic_map8()
    x = synth.normal(n, seed=9000 + seed, dtype=dtype, sigma=sigma)
    case(f"random config nested seed={seed} dtype={dtype} B={B} n={n} sigma={sigma:.3g}")
    packed, absmax = kb.quantize_kbit(to_dev(x, dtype), to_dev(cb), 4, B)
    code, a2, off = kb.quantize_nested_absmax(absmax, to_dev(q))
    torch.cuda.synchronize()
    want_w, want_a = kbit.quantize_packed(numerics.widen(x, dtype), cb, 4, B)
    assert_bits_equal(bits(packed), want_w, "words")
    assert_bits_equal(bits(absmax), np_bits(want_a), "absmax")
    wc, wa2, woff = nested.encode(want_a, q)
    assert bits(off)[0] == np.float32(woff).view(np.uint32), "offset"
    assert_bits_equal(bits(a2), np_bits(wa2), "absmax2")
    assert_bits_equal(bits(code), wc, "codes")
    out = kb.dequantize_4bit_nested(packed, to_dev(cb), code, to_dev(q), a2, float(np.float32(woff)), n,
                                    _tdt(dtype), B)
    torch.cuda.synchronize()
    want = nested.dequantize_packed(want_w, wc, wa2, np.float32(woff), q, cb, n, B, dtype)
    assert_bits_equal(bits(out), np_bits(want), "nested dequantize")


@pytest.mark.parametrize("seed", range(2100, 2124))
def test_random_config_quantize_to_nested(seed):
    # quantize_4bit_nested (the quantize kernel's exact sums, then the
    # encoder's second launch) against the oracle run from the input alone
    import torch
    from oracle import nested
    rng, dtype, _, B, n, kind, sigma = _config(seed)
    cb = codebooks.nf(4) if kind in ("nf", "unsorted") else _codebook(rng, "sorted", 4)
    q = codebooks.dynamic_map8()
    x = synth.normal(n, seed=9000 + seed, dtype=dtype, sigma=sigma)
    case(f"random config quantize to nested seed={seed} dtype={dtype} B={B} n={n} sigma={sigma:.3g}")
    packed, absmax, code, a2, off = kb.quantize_4bit_nested(to_dev(x, dtype), to_dev(cb), to_dev(q), B)
    torch.cuda.synchronize()
    want_w, want_a = kbit.quantize_packed(numerics.widen(x, dtype), cb, 4, B)
    assert_bits_equal(bits(packed), want_w, "words")
    assert_bits_equal(bits(absmax), np_bits(want_a), "absmax")
    wc, wa2, woff = nested.encode(want_a, q)
    assert bits(off)[0] == np.float32(woff).view(np.uint32), "offset"
    assert_bits_equal(bits(a2), np_bits(wa2), "absmax2")
    assert_bits_equal(bits(code), wc, "codes")


@pytest.mark.parametrize("seed", range(3000, 3040))
def test_random_config_activation(seed):
    # random width (a multiple of 256 up to 16384, so Hadamard blocks of
    # 256 .. 16384), row count, codebook scale and optional permutation
    from tests.test_gpu_act import check_act
    rng = np.random.default_rng(seed)
    d = 256 * int(rng.integers(1, 65))
    rows = int(rng.integers(1, 48))
    scale = float(2.0 ** rng.uniform(-6, 3))
    cb = (codebooks.lloyd_max_normal(16) * np.float32(scale)).astype(np.float32)
    x, s = synth.activations_bf16(tokens=rows, d=d, seed=seed)
    perm = rng.permutation(d) if rng.integers(2) else None
    check_act(x, s, cb, f"random seed={seed} scale={scale:.3g}", perm=perm)


@pytest.mark.parametrize("seed", range(3100, 3116))
def test_random_config_activation_prepared_tables(seed):
    # the same draw, through the codebook's prepared tables
    from tests.test_gpu_act_tables import check
    rng = np.random.default_rng(seed)
    d = 256 * int(rng.integers(1, 65))
    rows = int(rng.integers(1, 48))
    scale = float(2.0 ** rng.uniform(-6, 3))
    cb = (codebooks.lloyd_max_normal(16) * np.float32(scale)).astype(np.float32)
    x, s = synth.activations_bf16(tokens=rows, d=d, seed=seed)
    perm = rng.permutation(d) if rng.integers(2) else None
    check(x, s, cb, f"random seed={seed} scale={scale:.3g}", perm=perm)


@pytest.mark.parametrize("seed", range(4000, 4024))
def test_random_config_linear(seed):
    # random M, N, K (a multiple of 32) and blocksize; the fp32-sum bound of
    # the fused 4-bit linear against the exact products
    from oracle import linear
    from tests.test_gpu_linear import _check, _state, run_plain
    rng = np.random.default_rng(seed)
    M = int(rng.integers(1, 81))
    N = int(rng.integers(1, 201))
    K = 32 * int(rng.integers(1, 65))
    B = 1 << int(rng.integers(5, 9))
    case(f"random config linear seed={seed} M={M} N={N} K={K} B={B}")
    cb, words, absmax = _state(N, K, B, seed=seed)
    xb = synth.normal(M * K, seed=seed, dtype="bf16").reshape(M, K)
    got = run_plain(xb, words, cb, absmax, N, K, B)
    wb = linear.weights_bf16(words, cb, N, K, B, absmax=absmax)
    ref, absum = linear.reference(xb, wb)
    _check(got, ref, absum, K, f"random linear seed={seed}")
