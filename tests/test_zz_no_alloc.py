"""GPU check of quantize_nested_absmax_noalloc, the entry point for callers
that cannot allocate (its workspace is a static per-GPU array).

Called through the C ABI twice in a row, the second time on a smaller
input, and compared bit for bit with quantize_nested_absmax (caller-owned
workspace, filled with garbage first) on the same inputs; the small case
is also compared with the oracle.  Bar: bit-exact.
"""

import ctypes as ct

import numpy as np
import pytest

import blockwise_bit_codebook_amd as kb
from blockwise_bit_codebook_amd import synth
from oracle import codebooks, nested
from tests.gpu_util import assert_bits_equal, bits, case, np_bits, to_dev

pytestmark = pytest.mark.gpu


def _outputs(nb, dev):
    import torch
    return (torch.full((nb,), 0xAB, dtype=torch.uint8, device=dev),
            torch.full((-(-nb // 256),), float("nan"), dtype=torch.float32, device=dev),
            torch.full((1,), float("nan"), dtype=torch.float32, device=dev))


def _stream(dev):
    import torch
    return ct.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _p(t):
    return ct.c_void_p(t.data_ptr())


def _encode_both(a_np, q_np):
    import torch
    lib = kb.lib()
    a, q = to_dev(a_np), to_dev(q_np)
    dev = a.device
    nb = a.numel()
    code_r, a2_r, off_r = _outputs(nb, dev)
    ws = torch.full((lib.kbit_nested_workspace_bytes(nb),), 0x5A, dtype=torch.uint8, device=dev)
    assert lib.quantize_nested_absmax(_p(a), nb, _p(q), _p(code_r), _p(a2_r), _p(off_r), _p(ws), ws.numel(),
                                      _stream(dev)) == 0
    code_n, a2_n, off_n = _outputs(nb, dev)
    assert lib.quantize_nested_absmax_noalloc(_p(a), nb, _p(q), _p(code_n), _p(a2_n), _p(off_n), _stream(dev)) == 0
    torch.cuda.synchronize()
    return (bits(code_r), bits(a2_r), bits(off_r)), (bits(code_n), bits(a2_n), bits(off_n))


def _check(nb, seed, oracle=False):
    case(f"noalloc nested encode nb={nb} seed={seed}")
    a = np.abs(synth.normal(nb, seed=seed, dtype="fp32", sigma=0.05)).astype(np.float32)
    q = codebooks.dynamic_map8()
    ref, got = _encode_both(a, q)
    for r, g, what in zip(ref, got, ("codes", "absmax2", "offset")):
        assert_bits_equal(g, r, f"noalloc vs workspace entry point: {what} nb={nb}")
    if oracle:
        wc, wa2, woff = nested.encode(a, q)
        assert_bits_equal(got[0], wc, "noalloc codes vs oracle")
        assert_bits_equal(got[1], np_bits(wa2), "noalloc absmax2 vs oracle")
        assert got[2][0] == np.float32(woff).view(np.uint32)


def test_noalloc_matches_workspace_entry_point_twice():
    assert kb.lib().kbit_nested_noalloc_scratch_bytes() >= kb.lib().kbit_nested_workspace_bytes(1 << 36)
    _check(1048579, seed=21)             # 8192 x 8192 + 192 values at blocksize 64: 256 workgroups
    _check(5003, seed=22, oracle=True)   # then a smaller input on the same static workspace
    _check(5003, seed=23, oracle=True)   # and again
