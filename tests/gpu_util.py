"""Helpers for GPU parity tests: host<->device copies of raw bit patterns."""

import hashlib
import sys

import numpy as np

TORCH_DT = {"fp32": "float32", "fp16": "float16", "bf16": "bfloat16"}


def torch():
    import torch as _t
    return _t


def dev():
    return torch().device("cuda:0")


def to_dev(a, dtype=None):
    """numpy array -> CUDA tensor.  bf16 raw uint16 bits become a bfloat16 tensor."""
    t = torch()
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        return t.from_numpy(a.view(np.int16)).to(dev()).view(t.bfloat16)
    if a.dtype == np.uint32:
        return t.from_numpy(a.view(np.int32)).to(dev())
    if a.dtype == np.uint16:
        return t.from_numpy(a.view(np.int16)).to(dev())
    return t.from_numpy(a).to(dev())


def bits(tensor):
    """CUDA tensor -> numpy array of its raw bits (uint8/16/32)."""
    t = torch()
    h = tensor.detach().cpu()
    if h.dtype in (t.float32, t.int32):
        return h.view(t.int32).numpy().view(np.uint32)
    if h.dtype in (t.float16, t.bfloat16, t.int16):
        return h.view(t.int16).numpy().view(np.uint16)
    return h.numpy()


def np_bits(a):
    a = np.asarray(a)
    if a.dtype == np.float32:
        return a.view(np.uint32)
    if a.dtype == np.float16:
        return a.view(np.uint16)
    return a


def sha(tensor):
    return hashlib.sha256(tensor.detach().cpu().view(torch().uint8).numpy().tobytes()).hexdigest()


def case(msg):
    """Name the case on stderr before a GPU step (survives a lost box)."""
    print(f"[case] {msg}", file=sys.stderr, flush=True)


def assert_f32_bits_equal_nan_as_nan(got, want, what):
    """fp32 bit patterns equal, except that a NaN matches any NaN: IEEE
    754 leaves the sign and payload of a NaN result open when NaN operands
    meet, and the pages do not fix them; the NaN positions must match."""
    got = np.asarray(got, np.uint32)
    want = np.asarray(want, np.uint32)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    gnan = ((got & 0x7F800000) == 0x7F800000) & ((got & 0x7FFFFF) != 0)
    wnan = ((want & 0x7F800000) == 0x7F800000) & ((want & 0x7FFFFF) != 0)
    bad = np.flatnonzero(gnan != wnan)
    assert bad.size == 0, f"{what}: NaN at {bad[:5].tolist()} on one side only"
    assert_bits_equal(np.where(gnan, 0, got), np.where(wnan, 0, want), what)


def assert_bits_equal(got, want, what):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, f"{what}: {bad.size} mismatches, first at {bad[:5].tolist()}: got {got[bad[:5]]} want {want[bad[:5]]}"
