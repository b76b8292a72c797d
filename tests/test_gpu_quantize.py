"""GPU parity: blockwise quantize (absmax, packed bit planes) vs the oracle.

Bar: bit-exact.  Inputs are seeded synthetic arrays; near-threshold and
special-value cases are built by the test from the codebook values alone.
"""

import numpy as np
import pytest

import blockwise_bit_codebook_amd as kb
from blockwise_bit_codebook_amd import synth
from oracle import codebooks, kbit, numerics
from tests.gpu_util import assert_bits_equal, bits, case, np_bits, sha, to_dev

pytestmark = pytest.mark.gpu

DTYPES = ["fp32", "fp16", "bf16"]


def _cb(name, K):
    if name == "nf":
        return codebooks.nf(K)
    if name == "fp4":
        return codebooks.fp4()
    if name == "pages":
        return codebooks.nf_pages_rule(K)
    if name == "linspace":
        return np.linspace(-1, 1, 1 << K).astype(np.float32)
    if name == "dense":      # close distinct neighbours (1e-3), still on the threshold path
        c = codebooks.nf(K).copy()
        c[1] = c[0] + np.float32(1e-3)
        return c
    if name == "denser":     # neighbours 2^-20 apart (below the threshold path's 2^-16): full scan
        c = codebooks.nf(K).copy()
        c[1] = c[0] + np.float32(2.0 ** -20)
        return c
    if name == "unsorted":
        c = codebooks.nf(K).copy()[::-1].copy()
        return c
    if name == "wide":       # values outside [-1, 1]: exact path
        return (codebooks.nf(K) * np.float32(1.5)).astype(np.float32)
    raise ValueError(name)


def run_quantize(x_store, dtype, cb, K, B):
    A = to_dev(x_store, dtype)
    import torch
    packed, absmax = kb.quantize_kbit(A, to_dev(cb), K, B)
    torch.cuda.synchronize()
    return bits(packed), bits(absmax)


def check_quantize(x_store, dtype, cb, K, B, what):
    case(f"quantize {what} dtype={dtype} K={K} B={B} n={x_store.size}")
    words, absmax = run_quantize(x_store, dtype, cb, K, B)
    x32 = numerics.widen(x_store, dtype)
    want_w, want_a = kbit.quantize_packed(x32, cb, K, B)
    assert_bits_equal(absmax, np_bits(want_a), f"absmax {what}")
    assert_bits_equal(words, want_w, f"words {what}")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("K", [2, 3, 4, 5])
@pytest.mark.parametrize("B", [32, 64])
def test_small_sizes(dtype, K, B):
    for n in (1, 7, 31, 32, 33, 63, 64, 65, 511, 512, 513, 1000, 2047, 2048, 2049, 4097, 65613):
        x = synth.normal(n, seed=1000 + n + K, dtype=dtype)
        check_quantize(x, dtype, codebooks.nf(K), K, B, f"small n={n}")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("B", [32, 64, 128, 256, 512, 1024, 2048, 4096])
def test_block_sizes(dtype, B):
    n = 3 * 4096 * 8 + 1000
    x = synth.normal(n, seed=B, dtype=dtype)
    check_quantize(x, dtype, codebooks.nf(4), 4, B, "bsweep")
    check_quantize(x, dtype, codebooks.nf(3), 3, B, "bsweep")


@pytest.mark.parametrize("cbname,K", [("fp4", 4), ("pages", 4), ("pages", 2), ("linspace", 3), ("linspace", 5),
                                      ("nf", 5), ("dense", 4), ("denser", 4), ("unsorted", 3),
                                      ("wide", 4)])
def test_codebooks(cbname, K):
    x = synth.normal(50000, seed=7, dtype="bf16")
    check_quantize(x, "bf16", _cb(cbname, K), K, 64, cbname)


def _ulp_shift(v, steps):
    """float32 values moved by ``steps`` ulps along the real line (crossing zero)."""
    b = v.view(np.uint32).astype(np.int64)
    key = np.where(b < 0x80000000, b, -(b - 0x80000000)) + steps
    out = np.where(key >= 0, key, (-key) | 0x80000000).astype(np.uint32)
    return out.view(np.float32)


def _near_threshold_input(cb, B, nblocks, seed, jitter=8):
    """Blocks whose first element is the absmax a and whose other elements sit
    within a few ulps of (midpoint of neighbouring codes) * a."""
    rng = np.random.default_rng(seed)
    c = np.unique(cb.astype(np.float64))
    mids = (c[:-1] + c[1:]) / 2
    x = np.empty(nblocks * B, np.float32)
    for b in range(nblocks):
        a = np.float32(rng.uniform(0.01, 100.0))
        blk = np.empty(B, np.float32)
        blk[0] = a if rng.random() < 0.5 else -a
        m = np.float32(mids[rng.integers(0, mids.size, B - 1)])
        v = (m * a).astype(np.float32)
        steps = rng.integers(-jitter, jitter + 1, B - 1)
        blk[1:] = np.clip(_ulp_shift(v, steps), -a, a)
        x[b * B:(b + 1) * B] = blk
    return x


@pytest.mark.parametrize("cbname,K", [("nf", 2), ("nf", 3), ("nf", 4), ("nf", 5), ("fp4", 4), ("pages", 4)])
@pytest.mark.parametrize("B", [32, 64])
def test_near_thresholds_fp32(cbname, K, B):
    cb = _cb(cbname, K)
    x = _near_threshold_input(cb, B, 400, seed=K * 10 + B)
    check_quantize(x, "fp32", cb, K, B, f"near {cbname}")


def _near_threshold_16bit(cb, B, nblocks, dtype, seed, jitter=3):
    """16-bit blocks whose first element is the absmax a (a 16-bit value)
    and whose other elements are the 16-bit values within a few steps of
    (midpoint of neighbouring codes) * a: the inputs that decide each
    threshold by the narrowest margins."""
    rng = np.random.default_rng(seed)
    c = np.unique(cb.astype(np.float64))
    mids = (c[:-1] + c[1:]) / 2

    def to16(v):
        return numerics.to_bf16_bits(v) if dtype == "bf16" else numerics.to_fp16(v).view(np.uint16)

    out = np.empty(nblocks * B, np.uint16)
    for b in range(nblocks):
        a16 = to16(np.float32(rng.uniform(0.01, 100.0)))
        a = numerics.widen(np.array([a16], np.uint16) if dtype == "bf16" else np.array([a16]).view(np.float16),
                           dtype)[0]
        m = mids[rng.integers(0, mids.size, B - 1)]
        v = to16((m * np.float64(a)).astype(np.float32)).astype(np.int64)
        # step through neighbouring 16-bit values (sign-magnitude bits)
        steps = rng.integers(-jitter, jitter + 1, B - 1)
        mag = np.clip((v & 0x7FFF) + steps, 0, int(a16) & 0x7FFF)
        blk = ((v & 0x8000) | mag).astype(np.uint16)
        sign = 0x8000 if rng.random() < 0.5 else 0
        out[b * B] = np.uint16(int(a16) | sign)
        out[b * B + 1:(b + 1) * B] = blk
    return out if dtype == "bf16" else out.view(np.float16)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("cbname,K", [("nf", 2), ("nf", 3), ("nf", 4), ("nf", 5), ("fp4", 4), ("pages", 4),
                                      ("linspace", 4)])
def test_near_thresholds_16bit(dtype, cbname, K):
    # the fp32 two-fma threshold decision (16-bit inputs, K <= 4) and the fp64
    # one (K = 5) against the oracle's division, at the narrowest margins
    cb = _cb(cbname, K)
    x = _near_threshold_16bit(cb, 64, 600, dtype, seed=K * 7 + len(cbname))
    check_quantize(x, dtype, cb, K, 64, f"near16 {cbname}")


def test_tiny_blocks_16bit():
    # blocks with 0 < absmax < 1e-8 divide by the clamp 1e-8f (24 significant
    # bits), which the fp32 decision does not cover: they take the exact path;
    # all-zero blocks stay on the fast path
    cb = codebooks.nf(4)
    x = synth.normal(64 * 64, seed=5, dtype="fp32")
    for b in range(0, 64, 4):
        x[b * 64:(b + 1) * 64] *= np.float32(10.0 ** -(9 + b / 8))
    x[3 * 64:4 * 64] = 0.0
    xb = numerics.to_bf16_bits(x)
    check_quantize(xb, "bf16", cb, 4, 64, "tiny bf16")
    xh = numerics.to_fp16(x * np.float32(1e4))    # fp16 cannot hold 1e-9: scale into its subnormals
    check_quantize(xh, "fp16", cb, 4, 64, "tiny fp16")


def test_special_values():
    cb = codebooks.nf(4)
    x = synth.normal(64 * 40, seed=3, dtype="fp32")
    x[0:64] = 0.0                                   # all-zero block
    x[64:128] = -0.0                                # negative zeros
    x[128:192] *= np.float32(1e-41)                 # subnormal block, clamp 1e-8
    x[192:256] *= np.float32(1e-12)                 # tiny block below the clamp
    x[256:320] *= np.float32(3e37)                  # huge block (exact path)
    x[320:384] = np.float32(1e38)                   # constant huge
    x[384:448] *= np.float32(2e-38)                 # mixed normal/subnormal
    x[448] = np.float32(1e-45)
    check_quantize(x, "fp32", cb, 4, 64, "special")
    check_quantize(x.astype(np.float32), "fp32", codebooks.fp4(), 4, 32, "special fp4")
    xb = numerics.to_bf16_bits(x)
    check_quantize(xb, "bf16", cb, 4, 64, "special bf16")


def test_round_trip_config_fp32_65536():
    # 65,536 fp32 N(0,1), K=4 NF, blocksize 32
    x = synth.round_trip_fp32()
    check_quantize(x, "fp32", codebooks.nf(4), 4, 32, "config round trip")


@pytest.mark.parametrize("K", [2, 3, 4, 5])
def test_k_sweep_bf16_full(K):
    # 2^24 + 17 bf16 N(0,1) with 0.1% outliers x20, blocksize 32; every word checked
    x = synth.k_sweep_bf16()
    check_quantize(x, "bf16", codebooks.nf(K), K, 32, "k sweep")


@pytest.mark.parametrize("dtype", ["fp16", "fp32"])
@pytest.mark.parametrize("K", [2, 3, 5])
def test_k_sweep_fp16_fp32_blocksize64(dtype, K):
    # 2^22 + 77 N(0,1) elements, blocksize 64 (the configuration of the
    # input-type x K measurements); every word checked
    x = synth.normal((1 << 22) + 77, seed=500 + K, dtype=dtype)
    check_quantize(x, dtype, codebooks.nf(K), K, 64, f"k sweep {dtype}")


def test_determinism_and_input_immutability():
    import torch
    x = synth.k_sweep_bf16(n=(1 << 20) + 5)
    A = to_dev(x, "bf16")
    cb = to_dev(codebooks.nf(4))
    h0, hc = sha(A), sha(cb)
    p1, a1 = kb.quantize_kbit(A, cb, 4, 64)
    p2, a2 = kb.quantize_kbit(A, cb, 4, 64)
    torch.cuda.synchronize()
    assert sha(A) == h0 and sha(cb) == hc
    assert torch.equal(p1, p2) and torch.equal(a1.view(torch.int32), a2.view(torch.int32))


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_full_size_8192_square(dtype):
    # the measured workload: 8192 x 8192, N(0, 0.02), blocksize 64, NF4;
    # every word and every absmax compared with the oracle
    x = synth.weight(8192, 8192, dtype, seed=synth.SEED_WEIGHT_SHAPES)
    check_quantize(x, dtype, codebooks.nf(4), 4, 64, "8192^2")


def test_full_size_8192_square_fp4_bf16():
    # the FP4 side measurement's workload: 8192 x 8192 bf16, blocksize 64,
    # FP4 (whose simple midpoints many bf16 values hit exactly); in full
    x = synth.weight(8192, 8192, "bf16", seed=synth.SEED_WEIGHT_SHAPES)
    check_quantize(x, "bf16", codebooks.fp4(), 4, 64, "8192^2 fp4")


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("shape", ["wide11008", "tall11008", "square8192"])
def test_weight_shapes_with_tail(shape, dtype):
    # 11008 x 4096, 4096 x 11008 and 8192 x 8192 weights plus a 192-element
    # tail (three more blocks of 64), NF4, blocksize 64; in full
    rows, cols = synth.WEIGHT_SHAPES[shape]
    x = synth.weight(rows, cols, dtype, seed=synth.SEED_WEIGHT_SHAPES, extra=synth.TAIL_EXTRA)
    check_quantize(x, dtype, codebooks.nf(4), 4, 64, f"{shape}+{synth.TAIL_EXTRA}")
