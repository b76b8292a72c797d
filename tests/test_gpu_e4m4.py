"""GPU parity: k-bit quantize / dequantize with one-byte E4M4 block scales.

Bar: bit-exact against the oracle (``oracle.e4m4`` on top of ``oracle.kbit``).
Inputs are seeded synthetic arrays; scale edge cases (zero, E4M4 subnormals,
mantissa ties, binade tops, values above the range, inf, NaN) are built from
the format's own grid.
"""

import numpy as np
import pytest

import blockwise_bit_codebook_amd as kb
from blockwise_bit_codebook_amd import synth
from oracle import codebooks, e4m4, kbit, numerics
from tests.gpu_util import TORCH_DT, assert_bits_equal, bits, case, np_bits, to_dev

pytestmark = pytest.mark.gpu

DTYPES = ["fp32", "fp16", "bf16"]


def _tdt(dtype):
    import torch
    return getattr(torch, TORCH_DT[dtype])


def check_quantize(x_store, dtype, cb, K, B, what):
    import torch
    n = x_store.size
    case(f"quantize_e4m4 {what} dtype={dtype} K={K} B={B} n={n}")
    packed, code = kb.quantize_kbit(to_dev(x_store, dtype), to_dev(cb), K, B, absmax_format="e4m4")
    torch.cuda.synchronize()
    assert code.dtype == torch.uint8 and code.numel() == kb.n_blocks(n, B)
    want_w, want_c = e4m4.quantize_packed(numerics.widen(x_store, dtype), cb, K, B)
    assert_bits_equal(bits(code), want_c, f"codes {what}")
    assert_bits_equal(bits(packed), want_w, f"words {what}")


def check_dequant(idx, code, cb, K, B, dtype, what):
    import torch
    n = idx.size
    case(f"dequantize_e4m4 {what} dtype={dtype} K={K} B={B} n={n}")
    out = kb.dequantize_kbit(to_dev(kbit.pack(idx, K)), to_dev(cb), to_dev(code), K, n, _tdt(dtype), B)
    torch.cuda.synchronize()
    assert_bits_equal(bits(out), np_bits(e4m4.dequantize(idx, code, cb, B, dtype)), f"dequant {what}")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("K", [2, 3, 4, 5])
def test_quantize_small_sizes(dtype, K):
    for B in (32, 64):
        for n in (1, 31, 33, 64, 65, 511, 513, 2049, 65613):
            x = synth.normal(n, seed=3000 + n + K, dtype=dtype)
            check_quantize(x, dtype, codebooks.nf(K), K, B, f"small n={n}")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("B", [32, 64, 128, 256, 512, 1024, 2048, 4096])
def test_quantize_block_sizes(dtype, B):
    n = 3 * 4096 * 8 + 1000
    x = synth.normal(n, seed=B + 1, dtype=dtype)
    check_quantize(x, dtype, codebooks.nf(4), 4, B, "bsweep")


def _grid_edges():
    """Scales on and around the E4M4 grid: every code value, every midpoint
    between neighbours and the floats on either side, binade tops."""
    g = e4m4.decode(np.arange(256, dtype=np.uint8)).astype(np.float64)
    mids = (g[:-1] + g[1:]) / 2
    v = [g, mids]
    for m in mids:
        f = np.float32(m)
        v.append(np.array([np.nextafter(f, np.float32(0)), np.nextafter(f, np.float32(1e9))], np.float64))
    for e in range(-14, 8):
        f = np.float32(2.0 ** e)
        v.append(np.array([np.nextafter(f, np.float32(0))], np.float64))
    v.append(np.array([32.0, 100.0, 1e6, 3.4e38, 1e-45, 1e-40, 2.0 ** -126], np.float64))
    # and log-uniform draws over [2^-24, 2^8)
    v.append(np.exp2(np.random.default_rng(3).uniform(-24, 8, 20000)))
    return np.concatenate(v).astype(np.float32)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_quantize_scale_edges(dtype):
    # each block's absmax is a chosen edge value; the other elements are
    # smaller multiples of it with mixed signs
    amax = _grid_edges()
    if dtype == "bf16":
        amax = numerics.widen(numerics.to_bf16_bits(amax), "bf16")
    B = 32
    rng = np.random.default_rng(11)
    frac = rng.uniform(-1, 1, size=(amax.size, B)).astype(np.float32)
    x = (frac * amax[:, None]).astype(np.float32)
    pos = rng.integers(0, B, amax.size)
    x[np.arange(amax.size), pos] = amax * np.where(rng.random(amax.size) < 0.5, -1, 1).astype(np.float32)
    x = x.ravel()
    store = numerics.narrow(x, dtype)
    check_quantize(store, dtype, codebooks.nf(4), 4, B, "scale edges")


def test_quantize_special_blocks():
    # all-zero, +-inf and NaN blocks (fp32), with ordinary blocks around them
    B = 64
    x = synth.normal(B * 8, seed=21, dtype="fp32").reshape(8, B)
    x[1] = 0.0
    x[3, 5] = np.inf
    x[4, 7] = -np.inf
    x[6, 0] = np.nan
    xb = x.view(np.uint32)
    xb[7, 3] = 0x7F800001          # NaN payloads: signalling, and with the sign bit set
    xb[5, 9] = 0xFFC00123
    check_quantize(x.ravel().copy(), "fp32", codebooks.nf(3), 3, B, "special blocks")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("K", [2, 3, 4, 5])
def test_dequantize_all_codes(dtype, K):
    # every code byte appears as a block scale; ragged sizes
    B = 32
    for n in (1, 33, 512, 8191, 256 * 32 + 17):
        nb = kb.n_blocks(n, B)
        code = (np.arange(nb) * 37 % 256).astype(np.uint8)
        idx = synth.uniform_indices(n, K, seed=n + K)
        check_dequant(idx, code, codebooks.nf(K), K, B, dtype, f"codes n={n}")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("B", [32, 64, 128, 256, 512, 1024, 2048, 4096])
def test_dequantize_block_sizes(dtype, B):
    n = 5 * 4096 + 999
    idx = synth.uniform_indices(n, 4, seed=B + 7)
    code = np.random.default_rng(B).integers(0, 256, kb.n_blocks(n, B)).astype(np.uint8)
    for cb in (codebooks.nf(4), codebooks.fp4()):
        check_dequant(idx, code, cb, 4, B, dtype, "bsweep")


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_round_trip_weight_matrix(dtype):
    # 8192 x 8192 weight-like tensor, B = 64: quantize with E4M4 scales,
    # dequantize its own output; codes, words and outputs in full
    import torch
    rows = cols = 8192
    B, K = 64, 4
    x = synth.weight(rows, cols, dtype, seed=5)
    cb = codebooks.nf(K)
    case(f"e4m4 round trip {rows}x{cols} dtype={dtype}")
    packed, code = kb.quantize_kbit(to_dev(x, dtype), to_dev(cb), K, B, absmax_format="e4m4")
    out = kb.dequantize_kbit(packed, to_dev(cb), code, K, x.size, _tdt(dtype), B)
    torch.cuda.synchronize()
    n = x.size
    got_code, got_words, got_out = bits(code), bits(packed), bits(out)
    w, c = e4m4.quantize_packed(numerics.widen(x, dtype), cb, K, B)
    assert_bits_equal(got_code, c, "codes")
    assert_bits_equal(got_words, w, "words")
    want = e4m4.dequantize(kbit.unpack(w, K, n), c, cb, B, dtype)
    assert_bits_equal(got_out, np_bits(want), "out")
    assert got_code.size == kb.n_blocks(n, B) and got_words.size == kb.n_words(n, K)
