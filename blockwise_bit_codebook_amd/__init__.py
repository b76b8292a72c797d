"""MI355X-native blockwise absmax k-bit codebook quantization.

Thin Python binding over ``libkbit.so`` (C ABI in ``include/kbit.h``).  Every
step of the quantize / dequantize paths runs in the library's HIP kernels;
this module only allocates outputs with torch, checks tensor placement and
forwards raw device pointers and the current HIP stream.  If the library has
not been built, the first call raises ``ImportError``: there is no fallback.

Entry points carry the C names (``quantize_kbit_bf16_k4``,
``quantize_kbit_e4m4_bf16_k4``, ``dequantize_4bit_nested_fp16``, ...) and a
few dtype/K-dispatching conveniences (``quantize_kbit``, ``dequantize_kbit``,
``dequantize_4bit_nested``, ``quantize_act_fwht_k4_bf16``).  The block scales
are fp32 absmax values or, with ``absmax_format="e4m4"``, one E4M4 byte per
block (uint8 tensor).
"""

import ctypes as ct

import numpy as np

__all__ = [
    "KbitError", "lib", "codebook_nf", "codebook_fp4", "codebook_lloyd_max_normal",
    "dynamic_map8", "quantize_kbit", "dequantize_kbit", "dequantize_4bit_nested", "quantize_nested_absmax", "linear_4bit",
    "quantize_act_fwht_k4_bf16", "quantize_act_rpbh_k4_bf16", "n_words", "n_blocks",
]

_TORCH_NAME = {"fp32": "float32", "fp16": "float16", "bf16": "bfloat16"}


class KbitError(RuntimeError):
    """A libkbit entry point returned a non-zero status."""

    def __init__(self, fn, status, text):
        super().__init__(f"{fn}: {text} (status {status})")
        self.status = status


def lib():
    """The loaded ctypes library (raises ImportError if it was not built)."""
    from . import _lib
    return _lib.lib


def _check(fn_name, status):
    if status != 0:
        raise KbitError(fn_name, status, lib().kbit_strerror(status).decode())


def n_blocks(n, blocksize):
    return -(-n // blocksize)


def n_words(n, K):
    return -(-n // 32) * K


# --------------------------------------------------------------------------
# codebooks (host)
# --------------------------------------------------------------------------
def _host_table(fn_name, size, *args):
    out = np.zeros(size, dtype=np.float32)
    _check(fn_name, getattr(lib(), fn_name)(*args, out.ctypes.data_as(ct.c_void_p)))
    return out


def codebook_nf(K):
    return _host_table("kbit_codebook_nf", 1 << K, K)


def codebook_fp4():
    return _host_table("kbit_codebook_fp4", 16)


def codebook_lloyd_max_normal(levels=16):
    return _host_table("kbit_codebook_lloyd_max_normal", levels, levels)


def dynamic_map8():
    return _host_table("kbit_dynamic_map8", 256)


# --------------------------------------------------------------------------
# device entry points
# --------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _dtype_name(t):
    torch = _torch()
    for name, tn in _TORCH_NAME.items():
        if t == getattr(torch, tn):
            return name
    raise TypeError(f"unsupported element dtype {t}")


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return ct.c_void_p(t.data_ptr())


def _stream(device):
    torch = _torch()
    return ct.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _scale_infix(absmax_format):
    if absmax_format == "fp32":
        return ""
    if absmax_format == "e4m4":
        return "e4m4_"
    raise ValueError(f"absmax_format must be 'fp32' or 'e4m4', got {absmax_format!r}")


def quantize_kbit(A, codebook, k, blocksize, absmax=None, packed=None, absmax_format="fp32"):
    """Quantize A (fp32/fp16/bf16 CUDA tensor, any shape) -> (packed int32, absmax).

    absmax is fp32, or uint8 E4M4 codes with ``absmax_format="e4m4"``."""
    torch = _torch()
    t = _dtype_name(A.dtype)
    n = A.numel()
    infix = _scale_infix(absmax_format)
    if absmax is None:
        absmax = torch.empty(n_blocks(n, blocksize), dtype=torch.uint8 if infix else torch.float32,
                             device=A.device)
    if packed is None:
        packed = torch.empty(n_words(n, k), dtype=torch.int32, device=A.device)
    name = f"quantize_kbit_{infix}{t}_k{k}"
    fn = getattr(lib(), name)
    _check(name, fn(_ptr(codebook), _ptr(A), _ptr(absmax), _ptr(packed), n, blocksize, _stream(A.device)))
    return packed, absmax


def dequantize_kbit(packed, codebook, absmax, k, n, dtype, blocksize, out=None):
    """Dequantize bit-plane words -> tensor of n elements of ``dtype``.

    absmax: fp32 scales, or uint8 E4M4 codes (selects the E4M4 entry point)."""
    torch = _torch()
    t = _dtype_name(dtype)
    if absmax.dtype == torch.uint8:
        infix = "e4m4_"
    elif absmax.dtype == torch.float32:
        infix = ""
    else:
        raise TypeError(f"absmax must be float32 or uint8 (E4M4), got {absmax.dtype}")
    if out is None:
        out = torch.empty(n, dtype=dtype, device=packed.device)
    name = f"dequantize_kbit_{infix}{t}_k{k}"
    fn = getattr(lib(), name)
    _check(name, fn(_ptr(packed), _ptr(codebook), _ptr(absmax), _ptr(out), n, blocksize, _stream(packed.device)))
    return out


def dequantize_4bit_nested(packed, codebook16, absmax_code, qmap2, absmax2, offset, n, dtype, blocksize,
                           out=None):
    """Nested 4-bit dequantize with the scale rebuild fused into the decode."""
    torch = _torch()
    t = _dtype_name(dtype)
    if out is None:
        out = torch.empty(n, dtype=dtype, device=packed.device)
    name = f"dequantize_4bit_nested_{t}"
    fn = getattr(lib(), name)
    _check(name, fn(_ptr(packed), _ptr(codebook16), _ptr(absmax_code), _ptr(qmap2), _ptr(absmax2),
                    ct.c_float(float(offset)), _ptr(out), n, blocksize, _stream(packed.device)))
    return out


def quantize_nested_absmax(absmax, qmap2, absmax_code=None, absmax2=None, offset=None, workspace=None):
    """Nested state of fp32 per-block absmax -> (absmax_code u8, absmax2 fp32, offset fp32[1]).

    offset stays on the device; the workspace is allocated here unless given."""
    torch = _torch()
    nb = absmax.numel()
    dev = absmax.device
    if absmax_code is None:
        absmax_code = torch.empty(nb, dtype=torch.uint8, device=dev)
    if absmax2 is None:
        absmax2 = torch.empty(-(-nb // 256), dtype=torch.float32, device=dev)
    if offset is None:
        offset = torch.zeros(1, dtype=torch.float32, device=dev)
    need = lib().kbit_nested_workspace_bytes(nb)
    if need < 0:
        raise KbitError("kbit_nested_workspace_bytes", -1, "nb out of range")
    if workspace is None:
        workspace = torch.empty(max(need, 8), dtype=torch.uint8, device=dev)
    name = "quantize_nested_absmax"
    _check(name, lib().quantize_nested_absmax(_ptr(absmax), nb, _ptr(qmap2), _ptr(absmax_code), _ptr(absmax2),
                                              _ptr(offset), _ptr(workspace), workspace.numel(), _stream(dev)))
    return absmax_code, absmax2, offset


def linear_4bit(X, packed, codebook16, N, blocksize, absmax=None, absmax_code=None, qmap2=None, absmax2=None,
                offset=None, out=None):
    """out[M, N] = X[M, K] @ W[N, K]^T with W decoded from its 4-bit planes inside
    the kernel (bf16 in and out).  Scales: fp32 ``absmax``, or the nested state
    (``absmax_code``, ``qmap2``, ``absmax2``, ``offset``)."""
    torch = _torch()
    if X.dtype != torch.bfloat16 or X.dim() != 2:
        raise TypeError("X must be a 2-D bfloat16 tensor")
    M, K = X.shape
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=X.device)
    if absmax_code is not None:
        name = "linear_4bit_nested_bf16"
        status = lib().linear_4bit_nested_bf16(_ptr(X), M, K, _ptr(packed), _ptr(codebook16), _ptr(absmax_code),
                                               _ptr(qmap2), _ptr(absmax2), ct.c_float(float(offset)), N,
                                               blocksize, _ptr(out), _stream(X.device))
    else:
        name = "linear_kbit_bf16_k4"
        status = lib().linear_kbit_bf16_k4(_ptr(X), M, K, _ptr(packed), _ptr(codebook16), _ptr(absmax), N,
                                           blocksize, _ptr(out), _stream(X.device))
    _check(name, status)
    return out


def quantize_act_fwht_k4_bf16(X, sign_bits, codebook16, row_norm=None, packed=None, perm=None):
    """Token norm + sign flip + block FWHT (h = largest power of two dividing
    d) + Lloyd-Max assignment of bf16 [rows, d]; with ``perm`` (int32 [d])
    the columns are permuted first (quantize_act_rpbh_k4_bf16)."""
    torch = _torch()
    if X.dtype != torch.bfloat16 or X.dim() != 2:
        raise TypeError("X must be a 2-D bfloat16 tensor")
    rows, d = X.shape
    if row_norm is None:
        row_norm = torch.empty(rows, dtype=torch.float32, device=X.device)
    if packed is None:
        packed = torch.empty(n_words(rows * d, 4), dtype=torch.int32, device=X.device)
    if perm is None:
        name = "quantize_act_fwht_k4_bf16"
        status = lib().quantize_act_fwht_k4_bf16(_ptr(X), rows, d, _ptr(sign_bits), _ptr(codebook16),
                                                  _ptr(row_norm), _ptr(packed), _stream(X.device))
    else:
        if perm.dtype != torch.int32 or perm.numel() != d:
            raise TypeError("perm must be an int32 tensor of d entries")
        name = "quantize_act_rpbh_k4_bf16"
        status = lib().quantize_act_rpbh_k4_bf16(_ptr(X), rows, d, _ptr(perm), _ptr(sign_bits), _ptr(codebook16),
                                                  _ptr(row_norm), _ptr(packed), _stream(X.device))
    _check(name, status)
    return packed, row_norm


def quantize_act_rpbh_k4_bf16(X, perm, sign_bits, codebook16, row_norm=None, packed=None):
    """Column permutation, then quantize_act_fwht_k4_bf16's path."""
    return quantize_act_fwht_k4_bf16(X, sign_bits, codebook16, row_norm=row_norm, packed=packed, perm=perm)


def _make_named(fn_name, generic, **fixed):
    def f(*args, **kw):
        kw.update(fixed)
        return generic(*args, **kw)
    f.__name__ = fn_name
    f.__doc__ = f"{generic.__doc__} (fixed: {fixed})"
    return f


def _install_named():
    torch_dt = lambda t: getattr(_torch(), _TORCH_NAME[t])  # noqa: E731
    g = globals()
    for t in _TORCH_NAME:
        for k in (2, 3, 4, 5):
            g[f"quantize_kbit_{t}_k{k}"] = _make_named(
                f"quantize_kbit_{t}_k{k}", lambda A, codebook, blocksize, _k=k, **kw:
                quantize_kbit(A, codebook, _k, blocksize, **kw))
            g[f"dequantize_kbit_{t}_k{k}"] = _make_named(
                f"dequantize_kbit_{t}_k{k}", lambda packed, codebook, absmax, n, blocksize, _k=k, _t=t, **kw:
                dequantize_kbit(packed, codebook, absmax, _k, n, torch_dt(_t), blocksize, **kw))
            g[f"quantize_kbit_e4m4_{t}_k{k}"] = _make_named(
                f"quantize_kbit_e4m4_{t}_k{k}", lambda A, codebook, blocksize, _k=k, **kw:
                quantize_kbit(A, codebook, _k, blocksize, absmax_format="e4m4", **kw))
            g[f"dequantize_kbit_e4m4_{t}_k{k}"] = _make_named(
                f"dequantize_kbit_e4m4_{t}_k{k}",
                lambda packed, codebook, absmax_e4m4, n, blocksize, _k=k, _t=t, **kw:
                dequantize_kbit(packed, codebook, absmax_e4m4, _k, n, torch_dt(_t), blocksize, **kw))
        g[f"dequantize_4bit_nested_{t}"] = _make_named(
            f"dequantize_4bit_nested_{t}",
            lambda packed, codebook16, absmax_code, qmap2, absmax2, offset, n, blocksize, _t=t, **kw:
            dequantize_4bit_nested(packed, codebook16, absmax_code, qmap2, absmax2, offset, n,
                                   torch_dt(_t), blocksize, **kw))


_install_named()
