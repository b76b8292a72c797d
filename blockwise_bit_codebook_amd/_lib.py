"""ctypes loader for libkbit.so and signatures of every exported symbol.

Argument marshalling only.  If the library is missing the import of this
module raises, so no caller can silently fall back to another path.
"""

import ctypes as ct
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkbit.so")

DTYPES = ("fp32", "fp16", "bf16")
KS = (2, 3, 4, 5)

_p = ct.c_void_p
_i64 = ct.c_int64
_i32 = ct.c_int32
_f32 = ct.c_float


def _signatures():
    """(name, argtypes) for every C entry point declared in include/kbit.h."""
    sig = [
        ("kbit_strerror", [ct.c_int]),
        ("kbit_abi_version", []),
        ("kbit_codebook_nf", [ct.c_int, _p]),
        ("kbit_codebook_fp4", [_p]),
        ("kbit_codebook_lloyd_max_normal", [ct.c_int, _p]),
        ("kbit_dynamic_map8", [_p]),
        ("quantize_act_fwht_k4_bf16", [_p, _i64, _i32, _p, _p, _p, _p, _p]),
        ("quantize_act_rpbh_k4_bf16", [_p, _i64, _i32, _p, _p, _p, _p, _p, _p]),
        ("kbit_act_tables_bytes", []),
        ("act_tables_k4", [_p, _p, _p]),
        ("quantize_act_fwht_k4_bf16_tables", [_p, _i64, _i32, _p, _p, _p, _p, _p]),
        ("quantize_act_rpbh_k4_bf16_tables", [_p, _i64, _i32, _p, _p, _p, _p, _p, _p]),
        ("kbit_nested_workspace_bytes", [_i64]),
        ("linear_kbit_bf16_k4", [_p, _i64, _i32, _p, _p, _p, _i32, _i32, _p, _p]),
        ("linear_4bit_nested_bf16", [_p, _i64, _i32, _p, _p, _p, _p, _p, _f32, _i32, _i32, _p, _p]),
        ("linear_4bit_nested_bf16_offptr", [_p, _i64, _i32, _p, _p, _p, _p, _p, _p, _i32, _i32, _p, _p]),
        ("quantize_nested_absmax", [_p, _i64, _p, _p, _p, _p, _p, _i64, _p]),
        ("kbit_nested_noalloc_scratch_bytes", []),
        ("quantize_nested_absmax_noalloc", [_p, _i64, _p, _p, _p, _p, _p]),
        ("kbit_quantize_nested_workspace_bytes", []),
    ]
    for t in DTYPES:
        for k in KS:
            sig.append((f"quantize_kbit_{t}_k{k}", [_p, _p, _p, _p, _i64, _i32, _p]))
            sig.append((f"dequantize_kbit_{t}_k{k}", [_p, _p, _p, _p, _i64, _i32, _p]))
            sig.append((f"quantize_kbit_e4m4_{t}_k{k}", [_p, _p, _p, _p, _i64, _i32, _p]))
            sig.append((f"dequantize_kbit_e4m4_{t}_k{k}", [_p, _p, _p, _p, _i64, _i32, _p]))
        sig.append((f"dequantize_4bit_nested_{t}", [_p, _p, _p, _p, _p, _f32, _p, _i64, _i32, _p]))
        sig.append((f"dequantize_4bit_nested_{t}_offptr", [_p, _p, _p, _p, _p, _p, _p, _i64, _i32, _p]))
        sig.append((f"quantize_4bit_nested_{t}", [_p, _p, _p, _p, _p, _p, _p, _p, _i64, _i32, _p, _i64, _p]))
    return sig


SIGNATURES = _signatures()


def load(path=LIB_PATH):
    if not os.path.exists(path):
        raise ImportError(
            f"libkbit.so not found at {path}; build it with "
            "`python -m blockwise_bit_codebook_amd.build` (hipcc, gfx950)")
    lib = ct.CDLL(path)
    for name, args in SIGNATURES:
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = {"kbit_strerror": ct.c_char_p, "kbit_nested_workspace_bytes": ct.c_int64,
                      "kbit_nested_noalloc_scratch_bytes": ct.c_int64,
                      "kbit_quantize_nested_workspace_bytes": ct.c_int64,
                      "kbit_act_tables_bytes": ct.c_int64}.get(name, ct.c_int)
    return lib


lib = load()
