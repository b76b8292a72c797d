"""GPU parity: linear layer over 4-bit weights, decode fused into the MFMA
product, against the float64 reference on the oracle's decoded weights.

Bar: within the fp32-accumulation bound of ``oracle.linear.tolerance`` (the
classic summation bound with one fp32 ulp per addition) plus the bf16
output rounding; bit-exact where every partial sum is exact.  Weight states
are seeded host-side (oracle quantize for small shapes, random bit planes and
scales for the large ones).
"""

import numpy as np
import pytest

import blockwise_bit_codebook_amd as kb
from blockwise_bit_codebook_amd import synth
from oracle import codebooks, kbit, linear, nested, numerics
from tests.gpu_util import assert_bits_equal, bits, case, to_dev

pytestmark = pytest.mark.gpu


def _state(N, K, B, seed, quantize=True):
    cb = codebooks.nf(4)
    n = N * K
    if quantize:
        w = synth.weight(N, K, "fp32", seed=seed)
        words, absmax = kbit.quantize_packed(w, cb, 4, B)
    else:
        rng = np.random.default_rng(seed)
        words = kbit.pack(synth.uniform_indices(n, 4, seed=seed), 4)
        absmax = rng.uniform(0.01, 0.06, -(-n // B)).astype(np.float32)
    return cb, words, absmax


def _check(got_bits, ref, absum, K, what):
    got = numerics.widen(got_bits, "bf16").astype(np.float64)
    tol = linear.tolerance(absum, K)
    lim = tol + 2.0 ** -8 * (np.abs(ref) + tol)
    bad = np.argwhere(np.abs(got - ref) > lim)
    assert bad.size == 0, f"{what}: {len(bad)} outside the bound, first {bad[:3].tolist()}"


def run_plain(x_bits, words, cb, absmax, N, K, B):
    import torch
    X = to_dev(x_bits, "bf16").reshape(x_bits.shape)
    out = kb.linear_4bit(X, to_dev(words), to_dev(cb), N, B, absmax=to_dev(absmax))
    torch.cuda.synchronize()
    return bits(out).reshape(x_bits.shape[0], N)


@pytest.mark.parametrize("M,N,K,B", [(1, 16, 32, 32), (1, 17, 64, 64), (5, 48, 96, 32), (16, 64, 256, 64),
                                     (33, 100, 512, 128), (64, 40, 320, 64), (65, 24, 1024, 256),
                                     (130, 33, 64, 64), (7, 19, 4096, 4096)])
def test_plain_shapes(M, N, K, B):
    case(f"linear plain M={M} N={N} K={K} B={B}")
    cb, words, absmax = _state(N, K, B, seed=M + N + K)
    xb = synth.normal(M * K, seed=M * 7 + K, dtype="bf16").reshape(M, K)
    got = run_plain(xb, words, cb, absmax, N, K, B)
    wb = linear.weights_bf16(words, cb, N, K, B, absmax=absmax)
    ref, absum = linear.reference(xb, wb)
    _check(got, ref, absum, K, f"plain M={M} N={N} K={K}")


@pytest.mark.parametrize("M,N", [(1, 4096), (8, 4096), (32, 4096), (32, 11008)])
def test_nested_page_shapes(M, N):
    # the page's dequantize-plus-linear controls: K = 4096, B = 64
    import torch
    K, B = 4096, 64
    case(f"linear nested M={M} N={N} K={K}")
    cb, words, _ = _state(N, K, B, seed=N + M, quantize=False)
    nb = N * K // B
    code, a2, off = synth.nested_state_synthetic(nb, seed=M)
    q = codebooks.dynamic_map8()
    xb = synth.normal(M * K, seed=M, dtype="bf16").reshape(M, K)
    out = kb.linear_4bit(to_dev(xb, "bf16").reshape(M, K), to_dev(words), to_dev(cb), N, B,
                         absmax_code=to_dev(code), qmap2=to_dev(q), absmax2=to_dev(a2), offset=off)
    torch.cuda.synchronize()
    wb = linear.weights_bf16(words, cb, N, K, B, code=code, qmap2=q, absmax2=a2, offset=off)
    ref, absum = linear.reference(xb, wb)
    _check(bits(out).reshape(M, N), ref, absum, K, f"nested M={M} N={N}")


def test_exact_sums_bit_exact():
    # codebook k/8 with unit scales: weights and products are exact dyadics,
    # every partial sum is exact in fp32, so the output is RN_bf16 of the sum
    M, N, K, B = 24, 48, 2048, 64
    rng = np.random.default_rng(3)
    cb = (np.arange(-8, 8) / 8.0).astype(np.float32)
    idx = synth.uniform_indices(N * K, 4, seed=5)
    words = kbit.pack(idx, 4)
    absmax = np.ones(N * K // B, np.float32)
    xb = numerics.to_bf16_bits(rng.integers(-4, 5, (M, K)).astype(np.float32))
    case("linear exact sums")
    got = run_plain(xb, words, cb, absmax, N, K, B)
    wb = linear.weights_bf16(words, cb, N, K, B, absmax=absmax)
    ref, _ = linear.reference(xb, wb)
    assert_bits_equal(got.ravel(), numerics.to_bf16_bits(ref.astype(np.float32)).ravel(), "exact sums")


def test_adversarial_partial_sums():
    # every weight is 1 (NF4's top entry, unit scales), so each output is the
    # fp32 sum of an X row, and the rows are built so that partial sums
    # round: huge values that cancel around many small ones, magnitudes
    # walking over 2^-20 .. 2^20 with alternating signs, and runs of equal
    # values below a large one.  The outputs must stay inside the bound,
    # which assumes only a faithful rounding of each addition in the matrix
    # cores.
    M, N, K, B = 4, 32, 4096, 64
    rng = np.random.default_rng(12)
    cb = codebooks.nf(4)
    assert cb[15] == 1.0
    words = kbit.pack(np.full(N * K, 15, np.uint8), 4)
    absmax = np.ones(N * K // B, np.float32)
    x = np.ones((M, K), np.float32)
    x[0, 0], x[0, -1] = 2.0 ** 24, -(2.0 ** 24)
    x[1, 1::2] *= -1
    x[1] *= np.exp2(np.cumsum(rng.choice([-1, 1], K)).clip(-20, 20))
    x[2] = 1.0 + 2.0 ** -7
    x[2, ::512] = 2.0 ** 23
    x[3] = rng.choice([-1.0, 1.0], K) * np.exp2(rng.integers(-20, 21, K))
    xb = numerics.to_bf16_bits(x)
    case("linear adversarial partial sums")
    got = run_plain(xb, words, cb, absmax, N, K, B)
    wb = linear.weights_bf16(words, cb, N, K, B, absmax=absmax)
    ref, absum = linear.reference(xb, wb)
    _check(got, ref, absum, K, "adversarial")


def test_matches_dequantize_then_matmul():
    # the decoded operand is the dequantize kernel's output: decode with the
    # library, multiply in float64, compare within the same bound
    import torch
    M, N, K, B = 12, 64, 512, 64
    cb, words, absmax = _state(N, K, B, seed=9)
    xb = synth.normal(M * K, seed=10, dtype="bf16").reshape(M, K)
    case("linear vs dequantize")
    w_gpu = kb.dequantize_kbit(to_dev(words), to_dev(cb), to_dev(absmax), 4, N * K, torch.bfloat16, B)
    got = run_plain(xb, words, cb, absmax, N, K, B)
    torch.cuda.synchronize()
    wb = linear.weights_bf16(words, cb, N, K, B, absmax=absmax)
    assert_bits_equal(bits(w_gpu), wb.ravel(), "decoded weights")
    ref, absum = linear.reference(xb, wb)
    _check(got, ref, absum, K, "vs dequantize")
