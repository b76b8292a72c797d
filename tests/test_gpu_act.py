"""GPU parity: token norm + sign flip + FWHT + Lloyd-Max assignment (bit-exact)."""

import numpy as np
import pytest

import blockwise_bit_codebook_amd as kb
from blockwise_bit_codebook_amd import synth
from oracle import act, codebooks
from tests.gpu_util import assert_bits_equal, assert_f32_bits_equal_nan_as_nan, bits, case, np_bits, sha, to_dev

pytestmark = pytest.mark.gpu


def run_act(x, signs, cb, perm=None):
    import torch
    X = to_dev(x.reshape(-1), "bf16").view(x.shape[0], x.shape[1])
    P = None if perm is None else torch.from_numpy(np.asarray(perm, np.int32)).cuda()
    packed, norms = kb.quantize_act_fwht_k4_bf16(X, to_dev(signs), to_dev(cb), perm=P)
    torch.cuda.synchronize()
    return bits(packed), bits(norms)


def check_act(x, signs, cb, what, perm=None):
    case(f"act {what} rows={x.shape[0]} d={x.shape[1]} perm={perm is not None}")
    words, norms = run_act(x, signs, cb, perm)
    want_w, want_n = act.assign(x, signs, cb, perm=perm)
    assert_f32_bits_equal_nan_as_nan(norms, np_bits(want_n), f"norms {what}")
    assert_bits_equal(words, want_w, f"words {what}")


def test_small_rows():
    x, s = synth.activations_bf16(tokens=37, d=4096, seed=1)
    check_act(x, s, codebooks.lloyd_max_normal(16), "small")


def test_special_rows():
    x, s = synth.activations_bf16(tokens=8, d=4096, seed=2)
    x[0] = 0                                                   # zero row
    x[1] = 0
    x[1, 17] = 0x3F80                                          # single 1.0
    x[2] = (x[2].astype(np.uint32) & 0x807F).astype(np.uint16) | 0x0080   # tiny normals
    x[3] = (x[3] & 0x80FF) | 0x7E00                           # huge magnitudes
    x[4] = 0x3F80                                              # constant row
    x[5, 4000] = 0x7FC1                                        # NaN: the norm and every z are NaN
    check_act(x, s, codebooks.lloyd_max_normal(16), "special")


def test_other_codebook():
    x, s = synth.activations_bf16(tokens=16, d=4096, seed=3)
    cb = (codebooks.nf(4) * np.float32(2.5)).astype(np.float32)
    check_act(x, s, cb, "nf4 x 2.5")


def test_config_4096_tokens_full():
    # 4096 tokens x 4096 hidden, per-token log-uniform scale in [0.1, 10]
    x, s = synth.activations_bf16()
    check_act(x, s, codebooks.lloyd_max_normal(16), "config 4096x4096")


def test_immutability_and_determinism():
    import torch
    x, s = synth.activations_bf16(tokens=64, seed=4)
    X = to_dev(x.reshape(-1), "bf16").view(64, 4096)
    S, C = to_dev(s), to_dev(codebooks.lloyd_max_normal(16))
    h = [sha(X), sha(S), sha(C)]
    p1, n1 = kb.quantize_act_fwht_k4_bf16(X, S, C)
    p2, n2 = kb.quantize_act_fwht_k4_bf16(X, S, C)
    torch.cuda.synchronize()
    assert [sha(X), sha(S), sha(C)] == h
    assert torch.equal(p1, p2) and torch.equal(n1.view(torch.int32), n2.view(torch.int32))


# ---- block Hadamard (h = largest power of two dividing d), permutation ----

def scaled_lloyd_max(d):
    """The Lloyd-Max codebook scaled for d/h blocks (entries of z have about
    h/d of the variance they have for one block)."""
    h = act.hadamard_block(d)
    return (codebooks.lloyd_max_normal(16) * np.float32(np.sqrt(h / d))).astype(np.float32)


BLOCK_DIMS = [256, 768, 1536, 3072, 3840, 5120, 8192, 8960, 10240, 12288, 13824, 16128, 16384]


@pytest.mark.parametrize("d", BLOCK_DIMS)
def test_block_dims(d):
    x, s = synth.activations_bf16(tokens=37, d=d, seed=d)
    check_act(x, s, scaled_lloyd_max(d), "block")


@pytest.mark.parametrize("d", [768, 3840, 12288])
def test_block_dims_unscaled_codebook_and_few_rows(d):
    for rows in (1, 2, 5):
        x, s = synth.activations_bf16(tokens=rows, d=d, seed=rows + d)
        check_act(x, s, codebooks.lloyd_max_normal(16), "block unscaled")


@pytest.mark.parametrize("d", [256, 3840, 4096, 12288, 16384])
def test_permuted(d):
    x, s = synth.activations_bf16(tokens=21, d=d, seed=d + 1)
    perm = np.random.default_rng(d).permutation(d)
    check_act(x, s, scaled_lloyd_max(d), "rpbh", perm=perm)


def test_identity_permutation_matches_fixed_4096_kernel():
    # d = 4096 with a permutation runs the general kernel; with the identity
    # it must give what the dedicated d = 4096 kernel gives
    x, s = synth.activations_bf16(tokens=33, d=4096, seed=9)
    cb = codebooks.lloyd_max_normal(16)
    w0, n0 = run_act(x, s, cb)
    w1, n1 = run_act(x, s, cb, perm=np.arange(4096))
    assert_bits_equal(w1, w0, "identity perm words")
    assert_bits_equal(n1, n0, "identity perm norms")


@pytest.mark.parametrize("d", [3840, 12288])
def test_block_special_rows(d):
    x, s = synth.activations_bf16(tokens=8, d=d, seed=d + 2)
    x[0] = 0                                                   # zero row
    x[1] = 0
    x[1, d - 3] = 0x3F80                                       # single 1.0 in the last block
    x[2] = (x[2].astype(np.uint32) & 0x807F).astype(np.uint16) | 0x0080   # tiny normals
    x[3] = (x[3] & 0x80FF) | 0x7E00                           # huge magnitudes: norm overflows
    x[4] = 0x3F80                                              # constant row
    x[5, :256] = 0x7F80                                        # +inf in the first block
    x[6, 300] = 0x7FC1                                         # NaN
    check_act(x, s, scaled_lloyd_max(d), "block special")
    perm = np.random.default_rng(d).permutation(d)
    check_act(x, s, scaled_lloyd_max(d), "block special", perm=perm)


@pytest.mark.parametrize("d,rows", [(3840, 4096), (12288, 1024)])
def test_block_workloads_full(d, rows):
    # per-token log-uniform scale in [0.1, 10], as the d = 4096 workload
    x, s = synth.activations_bf16(tokens=rows, d=d, seed=d + 3)
    check_act(x, s, scaled_lloyd_max(d), "block workload")


@pytest.mark.parametrize("scale", [2.0 ** -12, 2.0 ** -5, 0.3, 3.0, 40.0])
def test_codebook_ranges(scale):
    # the bucket range follows the codebook's thresholds; narrow and wide
    # codebooks take the same exact decisions
    cb = (codebooks.lloyd_max_normal(16) * np.float32(scale)).astype(np.float32)
    for d in (4096, 8960):
        x, s = synth.activations_bf16(tokens=9, d=d, seed=int(d * scale) + 5)
        check_act(x, s, cb, f"codebook x {scale}")
