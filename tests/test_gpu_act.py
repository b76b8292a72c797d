"""GPU parity: token norm + sign flip + FWHT + Lloyd-Max assignment (bit-exact)."""

import numpy as np
import pytest

import blockwise_bit_codebook_amd as kb
from blockwise_bit_codebook_amd import synth
from oracle import act, codebooks
from tests.gpu_util import assert_bits_equal, bits, case, np_bits, sha, to_dev

pytestmark = pytest.mark.gpu


def run_act(x, signs, cb):
    import torch
    X = to_dev(x.reshape(-1), "bf16").view(x.shape[0], x.shape[1])
    packed, norms = kb.quantize_act_fwht_k4_bf16(X, to_dev(signs), to_dev(cb))
    torch.cuda.synchronize()
    return bits(packed), bits(norms)


def check_act(x, signs, cb, what):
    case(f"act {what} rows={x.shape[0]}")
    words, norms = run_act(x, signs, cb)
    want_w, want_n = act.assign(x, signs, cb)
    assert_bits_equal(norms, np_bits(want_n), f"norms {what}")
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
