"""Host-side checks of libkbit.so: exports, codebook generators, validation.

No compute call is made here; argument errors are detected by the library
before it touches a device.
"""

import ctypes as ct
import os
import re
import subprocess

import numpy as np
import pytest

from oracle import codebooks

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kbit.h")

kb = pytest.importorskip("blockwise_bit_codebook_amd")


def _lib():
    return kb.lib()


def _declared_functions():
    out = subprocess.run(["gcc", "-E", "-P", "-x", "c", HEADER], capture_output=True, text=True, check=True).stdout
    names = re.findall(r"\b(?:int|int64_t|const char\s*\*)\s+(\w+)\s*\(", out)
    return sorted(set(names))


def test_header_compiles_as_c_and_cpp():
    for lang in ("c", "c++"):
        subprocess.run(["gcc", "-fsyntax-only", "-Wall", "-Werror", "-x", lang, HEADER], check=True)


def test_every_declared_symbol_is_exported():
    names = _declared_functions()
    assert len(names) == 4 + 2 + 24 + 24 + 3 + 3 + 2 + 2 + 2 + 2 + 1 + 4 + 4, names
    nm = subprocess.run(["nm", "-D", "--defined-only", os.path.join(ROOT, "blockwise_bit_codebook_amd", "libkbit.so")],
                        capture_output=True, text=True, check=True).stdout
    exported = set(l.split()[-1] for l in nm.splitlines() if " T " in l)
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    from blockwise_bit_codebook_amd import _lib as L
    assert sorted(n for n, _ in L.SIGNATURES) == names


@pytest.mark.parametrize("K", [2, 3, 4, 5])
def test_nf_generator_equals_oracle(K):
    assert np.array_equal(kb.codebook_nf(K).view(np.uint32), codebooks.nf(K).view(np.uint32))


def test_fp4_generator_equals_oracle():
    assert np.array_equal(kb.codebook_fp4().view(np.uint32), codebooks.fp4().view(np.uint32))


def test_lloyd_max_generator_equals_oracle():
    assert np.array_equal(kb.codebook_lloyd_max_normal(16).view(np.uint32),
                          codebooks.lloyd_max_normal(16).view(np.uint32))


def test_dynamic_map_generator_equals_oracle():
    assert np.array_equal(kb.dynamic_map8().view(np.uint32), codebooks.dynamic_map8().view(np.uint32))


def test_generator_argument_errors():
    lib = _lib()
    buf = np.zeros(64, np.float32)
    p = buf.ctypes.data_as(ct.c_void_p)
    assert lib.kbit_codebook_nf(1, p) == -1
    assert lib.kbit_codebook_nf(6, p) == -1
    assert lib.kbit_codebook_nf(4, None) == -1
    assert lib.kbit_codebook_lloyd_max_normal(3, p) == -1
    assert lib.kbit_codebook_fp4(None) == -1
    assert lib.kbit_strerror(-2).decode().startswith("blocksize")
    assert lib.kbit_abi_version() == 3


# fake, never dereferenced device addresses
_A16 = ct.c_void_p(0x10000)
_A4 = ct.c_void_p(0x20004)


def test_validation_codes_before_any_device_access():
    lib = _lib()
    q = lib.quantize_kbit_bf16_k4
    assert q(_A16, _A16, _A16, _A16, 100, 48, None) == -2         # blocksize not power of two
    assert q(_A16, _A16, _A16, _A16, 100, 16, None) == -2         # too small
    assert q(_A16, _A16, _A16, _A16, 100, 8192, None) == -2       # too large
    assert q(_A16, _A16, _A16, _A16, -1, 64, None) == -1          # negative n
    assert q(_A16, _A16, _A16, _A16, (1 << 40) + 1, 64, None) == -1
    assert q(_A16, _A16, _A16, _A16, 0, 64, None) == 0            # empty: no-op
    assert q(None, None, None, None, 0, 64, None) == 0
    assert q(None, _A16, _A16, _A16, 10, 64, None) == -1          # null codebook
    assert q(_A16, _A4, _A16, _A16, 10, 64, None) == -3           # A not 16-byte aligned
    d = lib.dequantize_kbit_fp32_k3
    assert d(_A16, _A16, _A16, _A4, 10, 32, None) == -3           # out misaligned
    assert d(_A16, _A16, _A16, None, 10, 32, None) == -1
    nd = lib.dequantize_4bit_nested_fp16
    assert nd(_A16, _A16, None, _A16, _A16, ct.c_float(0.0), _A16, 10, 64, None) == -1
    assert nd(_A16, _A16, _A16, _A16, _A16, ct.c_float(0.0), _A16, 10, 96, None) == -2
    ndp = lib.dequantize_4bit_nested_fp16_offptr
    assert ndp(_A16, _A16, _A16, _A16, _A16, None, _A16, 10, 64, None) == -1      # no offset
    assert ndp(_A16, _A16, _A16, _A16, _A16, ct.c_void_p(0x20002), _A16, 10, 64, None) == -3  # offset misaligned
    assert ndp(None, None, None, None, None, None, None, 0, 64, None) == 0        # empty: no-op
    qe = lib.quantize_kbit_e4m4_fp16_k2
    _B1 = ct.c_void_p(0x30001)                                     # byte-aligned only
    assert qe(_A16, _A16, _B1, _A16, 10, 48, None) == -2
    assert qe(_A16, _A4, _B1, _A16, 10, 32, None) == -3           # A misaligned
    assert qe(_A16, _A16, None, _A16, 10, 32, None) == -1
    de = lib.dequantize_kbit_e4m4_bf16_k5
    assert de(_A16, _A16, _B1, _A4, 10, 64, None) == -3           # out misaligned
    assert de(_A16, _A16, None, _A16, 10, 64, None) == -1
    assert de(None, None, None, None, 0, 64, None) == 0
    assert lib.kbit_nested_workspace_bytes(0) == 0
    assert lib.kbit_nested_workspace_bytes(-1) == -1
    assert lib.kbit_nested_workspace_bytes((1 << 36) + 1) == -1
    wsb = lib.kbit_nested_workspace_bytes(1000)
    assert wsb >= 4 * 25                                       # one record of 25 32-bit words
    ne = lib.quantize_nested_absmax
    _W8 = ct.c_void_p(0x40000)
    assert ne(None, 0, None, None, None, None, None, 0, None) == 0                   # empty: no-op
    assert ne(_A16, -1, _A16, _A16, _A16, _A16, _W8, wsb, None) == -1
    assert ne(_A16, 1000, _A16, _A16, _A16, _A16, None, wsb, None) == -1          # no workspace
    assert ne(_A16, 1000, _A16, _A16, _A16, _A16, _W8, wsb - 1, None) == -1       # workspace too small
    assert ne(_A16, 1000, _A16, _A16, _A16, _A16, ct.c_void_p(0x40004), wsb, None) == -3
    assert ne(_A16, 1000, _A16, None, _A16, _A16, _W8, wsb, None) == -1
    assert ne(_A16, 1000, ct.c_void_p(0x20002), _A16, _A16, _A16, _W8, wsb, None) == -3
    qn = lib.quantize_4bit_nested_bf16
    qwb = lib.kbit_quantize_nested_workspace_bytes()
    assert qwb == 512 * 25 * 4                                    # one record per quantize workgroup
    assert qn(None, None, None, None, None, None, None, None, 0, 64, None, 0, None) == 0   # empty: no-op
    assert qn(_A16, _A16, _A16, _A16, _A16, _A16, _A16, _A16, 100, 48, _A16, qwb, None) == -2
    assert qn(_A16, _A16, _A16, _A16, _A16, _A16, _A16, _A16, -1, 64, _A16, qwb, None) == -1
    assert qn(_A16, _A16, _A16, _A16, _A16, _A16, _A16, _A16, 100, 64, None, qwb, None) == -1        # no workspace
    assert qn(_A16, _A16, _A16, _A16, _A16, _A16, _A16, _A16, 100, 64, _A16, qwb - 1, None) == -1    # too small
    assert qn(_A16, _A16, _A16, _A16, None, _A16, _A16, _A16, 100, 64, _A16, qwb, None) == -1        # no qmap2
    assert qn(_A16, _A16, _A16, _A16, _A16, _A16, _A16, None, 100, 64, _A16, qwb, None) == -1        # no offset
    assert qn(_A16, _A4, _A16, _A16, _A16, _A16, _A16, _A16, 100, 64, _A16, qwb, None) == -3         # A misaligned
    assert qn(_A16, _A16, ct.c_void_p(0x20002), _A16, _A16, _A16, _A16, _A16, 100, 64, _A16, qwb, None) == -3
    assert qn(_A16, _A16, _A16, _A16, _A16, _A16, _A16, _A16, 100, 64, ct.c_void_p(0x40002), qwb, None) == -3
    na = lib.quantize_nested_absmax_noalloc
    assert lib.kbit_nested_noalloc_scratch_bytes() >= lib.kbit_nested_workspace_bytes(1 << 36)
    assert na(None, 0, None, None, None, None, None) == 0                           # empty: no-op
    assert na(_A16, -1, _A16, _A16, _A16, _A16, None) == -1
    assert na(_A16, (1 << 36) + 1, _A16, _A16, _A16, _A16, None) == -1               # beyond the static workspace
    assert na(None, 1000, _A16, _A16, _A16, _A16, None) == -1
    assert na(_A16, 1000, _A16, _A16, _A16, None, None) == -1                        # no offset output
    assert na(_A16, 1000, ct.c_void_p(0x20002), _A16, _A16, _A16, None) == -3        # qmap2 misaligned
    li = lib.linear_kbit_bf16_k4
    assert li(_A16, 4, 48, _A16, _A16, _A16, 64, 64, _A16, None) == -1            # K not a multiple of 32
    assert li(_A16, 4, 64, _A16, _A16, _A16, 0, 64, _A16, None) == -1             # N = 0
    assert li(_A16, 4, 64, _A16, _A16, _A16, 64, 96, _A16, None) == -2            # blocksize
    assert li(None, 0, 64, None, None, None, 64, 64, None, None) == 0              # M = 0: no-op
    assert li(_A16, 4, 64, _A4, _A16, _A16, 64, 64, _A16, None) == -3             # packed not 16-byte aligned
    assert li(_A16, 4, 64, _A16, _A16, None, 64, 64, _A16, None) == -1            # no absmax
    ln = lib.linear_4bit_nested_bf16
    assert ln(_A16, 4, 64, _A16, _A16, None, _A16, _A16, ct.c_float(0), 64, 64, _A16, None) == -1
    lnp = lib.linear_4bit_nested_bf16_offptr
    assert lnp(_A16, 4, 64, _A16, _A16, _A16, _A16, _A16, None, 64, 64, _A16, None) == -1       # no offset
    assert lnp(_A16, 4, 64, _A16, _A16, _A16, _A16, _A16, ct.c_void_p(0x20002), 64, 64, _A16, None) == -3
    assert ln(_A4, 4, 64, _A16, _A16, _A16, _A16, _A16, ct.c_float(0), 64, 64, _A16, None) == -3
    act = lib.quantize_act_fwht_k4_bf16
    assert act(_A16, 4, 2000, _A16, _A16, _A16, _A16, None) == -1  # d not a multiple of 256
    assert act(_A16, 4, 128, _A16, _A16, _A16, _A16, None) == -1   # d below 256
    assert act(_A16, 4, 16640, _A16, _A16, _A16, _A16, None) == -1  # d above 16384
    assert act(_A16, 1 << 40, 4096, _A16, _A16, _A16, _A16, None) == -1  # rows * d too large
    assert act(_A16, 0, 4096, None, None, None, None, None) == 0
    assert act(_A4, 4, 4096, _A16, _A16, _A16, _A16, None) == -3
    rp = lib.quantize_act_rpbh_k4_bf16
    assert rp(_A16, 4, 3840, None, _A16, _A16, _A16, _A16, None) == -1   # no permutation
    assert rp(_A16, 4, 3900, _A16, _A16, _A16, _A16, _A16, None) == -1   # d
    assert rp(_A16, 4, 3840, _A4, _A16, _A16, _A16, _A16, None) == -3    # perm not 16-byte aligned
    assert rp(None, 0, 3840, None, None, None, None, None, None) == 0     # rows = 0: no-op
    assert lib.kbit_act_tables_bytes() == 133 * 16
    tb = lib.act_tables_k4
    assert tb(None, _A16, None) == -1                                    # no codebook
    assert tb(_A16, None, None) == -1                                    # no tables
    assert tb(_A16, _A4, None) == -3                                     # tables not 16-byte aligned
    at = lib.quantize_act_fwht_k4_bf16_tables
    assert at(_A16, 4, 4096, _A16, None, _A16, _A16, None) == -1         # no tables
    assert at(_A16, 4, 4096, _A16, _A4, _A16, _A16, None) == -3          # tables misaligned
    assert at(_A16, 4, 2000, _A16, _A16, _A16, _A16, None) == -1         # d
    assert at(None, 0, 4096, None, None, None, None, None) == 0
    rt = lib.quantize_act_rpbh_k4_bf16_tables
    assert rt(_A16, 4, 3840, None, _A16, _A16, _A16, _A16, None) == -1   # no permutation
    assert rt(_A16, 4, 3840, _A16, _A16, _A4, _A16, _A16, None) == -3    # tables misaligned
    assert rt(None, 0, 3840, None, None, None, None, None, None) == 0
