"""GPU parity of the activation path with prepared tables (act_tables_k4,
then the _tables entry points): bit-exact against the oracle, and equal to
the plain calls that build the tables in every workgroup."""

import numpy as np
import pytest

import blockwise_bit_codebook_amd as kb
from blockwise_bit_codebook_amd import synth
from oracle import act, codebooks
from tests.gpu_util import assert_bits_equal, assert_f32_bits_equal_nan_as_nan, bits, case, np_bits, to_dev

pytestmark = pytest.mark.gpu


def scaled_lloyd_max(d):
    h = act.hadamard_block(d)
    return (codebooks.lloyd_max_normal(16) * np.float32(np.sqrt(h / d))).astype(np.float32)


def run(x, signs, cb=None, tables=None, perm=None):
    import torch
    X = to_dev(x.reshape(-1), "bf16").view(x.shape[0], x.shape[1])
    P = None if perm is None else torch.from_numpy(np.asarray(perm, np.int32)).cuda()
    packed, norms = kb.quantize_act_fwht_k4_bf16(X, to_dev(signs), None if cb is None else to_dev(cb), perm=P,
                                                 tables=tables)
    torch.cuda.synchronize()
    return bits(packed), bits(norms)


def check(x, s, cb, what, perm=None):
    case(f"act tables {what} rows={x.shape[0]} d={x.shape[1]} perm={perm is not None}")
    tables = kb.act_tables_k4(to_dev(cb))
    words, norms = run(x, s, tables=tables, perm=perm)
    want_w, want_n = act.assign(x, s, cb, perm=perm)
    assert_f32_bits_equal_nan_as_nan(norms, np_bits(want_n), f"norms {what}")
    assert_bits_equal(words, want_w, f"words {what}")


@pytest.mark.parametrize("d", [4096, 256, 3840, 12288])
@pytest.mark.parametrize("permuted", [False, True])
def test_tables_match_oracle(d, permuted):
    x, s = synth.activations_bf16(tokens=29, d=d, seed=d + 11)
    perm = np.random.default_rng(d + 1).permutation(d) if permuted else None
    check(x, s, scaled_lloyd_max(d), "dims", perm=perm)


def test_tables_special_rows():
    x, s = synth.activations_bf16(tokens=8, d=4096, seed=12)
    x[0] = 0
    x[1, 17] = 0x3F80
    x[3] = (x[3] & 0x80FF) | 0x7E00                           # huge magnitudes
    x[5, 4000] = 0x7FC1                                        # NaN row: every index 0
    x[6, :256] = 0x7F80                                        # +inf
    check(x, s, codebooks.lloyd_max_normal(16), "special")


@pytest.mark.parametrize("name", ["nf4 x 2.5", "close entries", "unsorted"])
def test_tables_other_codebooks(name):
    # codebooks that take the fast path with another range, and two that do
    # not qualify for it (the exact path reads the codebook copy in the tables)
    cb = codebooks.lloyd_max_normal(16).copy()
    if name == "nf4 x 2.5":
        cb = (codebooks.nf(4) * np.float32(2.5)).astype(np.float32)
    elif name == "close entries":
        cb[8] = np.float32(cb[7] + np.float32(2.0 ** -14))
    else:
        cb = cb[::-1].copy()
    for d in (4096, 3840):
        x, s = synth.activations_bf16(tokens=11, d=d, seed=d + 13)
        check(x, s, cb, name)


def test_tables_rebuilt_in_place_follow_stream_order():
    import torch
    x, s = synth.activations_bf16(tokens=16, d=4096, seed=14)
    cb1 = codebooks.lloyd_max_normal(16)
    cb2 = (codebooks.nf(4) * np.float32(2.0)).astype(np.float32)
    X = to_dev(x.reshape(-1), "bf16").view(16, 4096)
    S = to_dev(s)
    tables = kb.act_tables_k4(to_dev(cb1))
    p1, n1 = kb.quantize_act_fwht_k4_bf16(X, S, tables=tables)
    kb.act_tables_k4(to_dev(cb2), tables=tables)               # same buffer, next on the stream
    p2, n2 = kb.quantize_act_fwht_k4_bf16(X, S, tables=tables)
    torch.cuda.synchronize()
    for p, cb in ((p1, cb1), (p2, cb2)):
        want_w, _ = act.assign(x, s, cb)
        assert_bits_equal(bits(p), want_w, "rebuilt tables")


@pytest.mark.parametrize("d,rows", [(4096, 4096), (3840, 4096)])
def test_tables_full_workload_equals_plain_call(d, rows):
    # the plain call is compared with the oracle at these sizes elsewhere
    x, s = synth.activations_bf16(tokens=rows, d=d, seed=d + 15)
    cb = scaled_lloyd_max(d)
    case(f"act tables full rows={rows} d={d}")
    w0, n0 = run(x, s, cb=cb)
    import torch
    tables = kb.act_tables_k4(to_dev(cb))
    w1, n1 = run(x, s, tables=tables)
    assert_bits_equal(w1, w0, "full words")
    assert_bits_equal(n1, n0, "full norms")
