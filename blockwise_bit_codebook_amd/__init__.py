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
import operator

import numpy as np

__all__ = [
    "KbitError", "lib", "codebook_nf", "codebook_fp4", "codebook_lloyd_max_normal",
    "dynamic_map8", "quantize_kbit", "dequantize_kbit", "dequantize_4bit_nested", "quantize_nested_absmax",
    "quantize_nested_absmax_noalloc", "quantize_4bit_nested", "linear_4bit",
    "quantize_act_fwht_k4_bf16", "quantize_act_rpbh_k4_bf16", "act_tables_k4", "n_words", "n_blocks",
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


def _buf(t, what, dtype, count):
    """Checks a buffer before its address goes to the library, which cannot
    check sizes or element types: the dtype, and at least ``count``
    elements.  Placement and contiguity are checked by ``_ptr``."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what}: expected a tensor, got {type(t).__name__}")
    if t.dtype != dtype:
        raise TypeError(f"{what}: element type {t.dtype}, expected {dtype}")
    if t.numel() < count:
        raise ValueError(f"{what}: {t.numel()} elements, at least {count} needed")
    return t


def _same_device(ref, **tensors):
    for what, t in tensors.items():
        if t is not None and t.device != ref.device:
            raise ValueError(f"{what} is on {t.device}, the input on {ref.device}")


def _blocks(n, blocksize):
    try:
        n, b = operator.index(n), operator.index(blocksize)
    except TypeError:
        raise TypeError(f"n and blocksize must be integers, got {n!r}, {blocksize!r}") from None
    if b <= 0:
        raise ValueError(f"blocksize must be positive, got {b}")
    if n < 0:
        raise ValueError(f"n must be >= 0, got {n}")
    return n_blocks(n, b)


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
    if k not in (2, 3, 4, 5):
        raise ValueError(f"k must be 2..5, got {k!r}")
    nb = _blocks(n, blocksize)
    sdt = torch.uint8 if infix else torch.float32
    if absmax is None:
        absmax = torch.empty(nb, dtype=sdt, device=A.device)
    if packed is None:
        packed = torch.empty(n_words(n, k), dtype=torch.int32, device=A.device)
    _buf(codebook, "codebook", torch.float32, 1 << k)
    _buf(absmax, "absmax (E4M4 bytes)" if infix else "absmax", sdt, nb)
    _buf(packed, "packed", torch.int32, n_words(n, k))
    _same_device(A, codebook=codebook, absmax=absmax, packed=packed)
    name = f"quantize_kbit_{infix}{t}_k{k}"
    fn = getattr(lib(), name)
    _check(name, fn(_ptr(codebook), _ptr(A), _ptr(absmax), _ptr(packed), n, blocksize, _stream(A.device)))
    return packed, absmax


def dequantize_kbit(packed, codebook, absmax, k, n, dtype, blocksize, out=None):
    """Dequantize bit-plane words -> tensor of n elements of ``dtype``.

    absmax: fp32 scales, or uint8 E4M4 codes (selects the E4M4 entry point)."""
    torch = _torch()
    t = _dtype_name(dtype)
    if k not in (2, 3, 4, 5):
        raise ValueError(f"k must be 2..5, got {k!r}")
    nb = _blocks(n, blocksize)
    if absmax.dtype == torch.uint8:
        infix = "e4m4_"
    elif absmax.dtype == torch.float32:
        infix = ""
    else:
        raise TypeError(f"dequantize_kbit: the block scales are a float32 tensor, or a uint8 tensor of "
                        f"E4M4 bytes; this one holds {absmax.dtype}")
    if out is None:
        out = torch.empty(n, dtype=dtype, device=packed.device)
    _buf(packed, "packed", torch.int32, n_words(n, k))
    _buf(codebook, "codebook", torch.float32, 1 << k)
    _buf(absmax, "absmax", absmax.dtype, nb)
    _buf(out, "out", dtype, n)
    _same_device(packed, codebook=codebook, absmax=absmax, out=out)
    name = f"dequantize_kbit_{infix}{t}_k{k}"
    fn = getattr(lib(), name)
    _check(name, fn(_ptr(packed), _ptr(codebook), _ptr(absmax), _ptr(out), n, blocksize, _stream(packed.device)))
    return out


def _nested_state(packed, codebook16, absmax_code, qmap2, absmax2, n, nb):
    torch = _torch()
    _buf(packed, "packed", torch.int32, n_words(n, 4))
    _buf(codebook16, "codebook16", torch.float32, 16)
    _buf(absmax_code, "absmax_code", torch.uint8, nb)
    _buf(qmap2, "qmap2", torch.float32, 256)
    _buf(absmax2, "absmax2", torch.float32, -(-nb // 256))
    _same_device(packed, codebook16=codebook16, absmax_code=absmax_code, qmap2=qmap2, absmax2=absmax2)


def dequantize_4bit_nested(packed, codebook16, absmax_code, qmap2, absmax2, offset, n, dtype, blocksize,
                           out=None):
    """Nested 4-bit dequantize with the scale rebuild fused into the decode.

    offset: a float, or a one-element float32 tensor on the device (such as
    quantize_nested_absmax's offset output), which the kernel reads itself."""
    torch = _torch()
    t = _dtype_name(dtype)
    nb = _blocks(n, blocksize)
    if out is None:
        out = torch.empty(n, dtype=dtype, device=packed.device)
    _nested_state(packed, codebook16, absmax_code, qmap2, absmax2, n, nb)
    _buf(out, "out", dtype, n)
    _same_device(packed, out=out)
    if isinstance(offset, torch.Tensor):
        # read on the device when the kernel starts: no host round trip
        _buf(offset, "offset", torch.float32, 1)
        _same_device(packed, offset=offset)
        name = f"dequantize_4bit_nested_{t}_offptr"
        off_arg = _ptr(offset)
    else:
        name = f"dequantize_4bit_nested_{t}"
        off_arg = ct.c_float(float(offset))
    fn = getattr(lib(), name)
    _check(name, fn(_ptr(packed), _ptr(codebook16), _ptr(absmax_code), _ptr(qmap2), _ptr(absmax2),
                    off_arg, _ptr(out), n, blocksize, _stream(packed.device)))
    return out


def _encode_args(absmax, qmap2, absmax_code, absmax2, offset):
    torch = _torch()
    nb = absmax.numel()
    _buf(absmax, "absmax", torch.float32, 0)
    _buf(qmap2, "qmap2", torch.float32, 256)
    _buf(absmax_code, "absmax_code", torch.uint8, nb)
    _buf(absmax2, "absmax2", torch.float32, -(-nb // 256))
    _buf(offset, "offset", torch.float32, 1)
    _same_device(absmax, qmap2=qmap2, absmax_code=absmax_code, absmax2=absmax2, offset=offset)


def quantize_nested_absmax(absmax, qmap2, absmax_code=None, absmax2=None, offset=None, workspace=None):
    """Nested state of fp32 per-block absmax -> (absmax_code u8, absmax2 fp32, offset fp32[1]).

    offset stays on the device; the workspace (scratch) is allocated here
    unless given."""
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
    _encode_args(absmax, qmap2, absmax_code, absmax2, offset)
    _buf(workspace, "workspace", torch.uint8, need)
    _same_device(absmax, workspace=workspace)
    name = "quantize_nested_absmax"
    _check(name, lib().quantize_nested_absmax(_ptr(absmax), nb, _ptr(qmap2), _ptr(absmax_code), _ptr(absmax2),
                                              _ptr(offset), _ptr(workspace), workspace.numel(), _stream(dev)))
    return absmax_code, absmax2, offset


def quantize_nested_absmax_noalloc(absmax, qmap2, absmax_code, absmax2, offset):
    """quantize_nested_absmax into caller-given outputs, with the library's
    static per-GPU workspace: no allocation.  Calls on one GPU must not
    overlap."""
    nb = absmax.numel()
    _encode_args(absmax, qmap2, absmax_code, absmax2, offset)
    name = "quantize_nested_absmax_noalloc"
    _check(name, lib().quantize_nested_absmax_noalloc(_ptr(absmax), nb, _ptr(qmap2), _ptr(absmax_code),
                                                      _ptr(absmax2), _ptr(offset), _stream(absmax.device)))
    return absmax_code, absmax2, offset


def quantize_4bit_nested(A, codebook16, qmap2, blocksize, absmax=None, packed=None, absmax_code=None,
                         absmax2=None, offset=None, workspace=None):
    """Quantize A (fp32/fp16/bf16 CUDA tensor) straight to the nested 4-bit
    state in two kernels -> (packed int32, absmax fp32, absmax_code u8,
    absmax2 fp32, offset fp32[1]); the same bits as quantize_kbit(A, ..., 4)
    followed by quantize_nested_absmax on its absmax.  The workspace
    (scratch) is allocated here unless given."""
    torch = _torch()
    t = _dtype_name(A.dtype)
    n = A.numel()
    nb = _blocks(n, blocksize)
    dev = A.device
    if absmax is None:
        absmax = torch.empty(nb, dtype=torch.float32, device=dev)
    if packed is None:
        packed = torch.empty(n_words(n, 4), dtype=torch.int32, device=dev)
    if absmax_code is None:
        absmax_code = torch.empty(nb, dtype=torch.uint8, device=dev)
    if absmax2 is None:
        absmax2 = torch.empty(-(-nb // 256), dtype=torch.float32, device=dev)
    if offset is None:
        offset = torch.zeros(1, dtype=torch.float32, device=dev)
    need = lib().kbit_quantize_nested_workspace_bytes()
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _buf(codebook16, "codebook16", torch.float32, 16)
    _buf(absmax, "absmax", torch.float32, nb)
    _buf(packed, "packed", torch.int32, n_words(n, 4))
    _encode_args(absmax, qmap2, absmax_code, absmax2, offset)
    _buf(workspace, "workspace", torch.uint8, need)
    _same_device(A, codebook16=codebook16, absmax=absmax, packed=packed, qmap2=qmap2, workspace=workspace)
    name = f"quantize_4bit_nested_{t}"
    fn = getattr(lib(), name)
    _check(name, fn(_ptr(codebook16), _ptr(A), _ptr(absmax), _ptr(packed), _ptr(qmap2), _ptr(absmax_code),
                    _ptr(absmax2), _ptr(offset), n, blocksize, _ptr(workspace), workspace.numel(), _stream(dev)))
    return packed, absmax, absmax_code, absmax2, offset


def linear_4bit(X, packed, codebook16, N, blocksize, absmax=None, absmax_code=None, qmap2=None, absmax2=None,
                offset=None, out=None):
    """out[M, N] = X[M, K] @ W[N, K]^T with W decoded from its 4-bit planes inside
    the kernel (bf16 in and out).  Scales: fp32 ``absmax``, or the nested state
    (``absmax_code``, ``qmap2``, ``absmax2``, ``offset`` as a float or a
    one-element float32 device tensor read by the kernel)."""
    torch = _torch()
    if X.dtype != torch.bfloat16 or X.dim() != 2:
        raise TypeError("X must be a 2-D bfloat16 tensor")
    M, K = X.shape
    nb = _blocks(N * K, blocksize)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=X.device)
    _buf(out, "out", torch.bfloat16, M * N)
    _same_device(X, out=out)
    if absmax_code is not None:
        _nested_state(packed, codebook16, absmax_code, qmap2, absmax2, N * K, nb)
        _same_device(X, packed=packed)
    else:
        _buf(packed, "packed", torch.int32, n_words(N * K, 4))
        _buf(codebook16, "codebook16", torch.float32, 16)
        _buf(absmax, "absmax", torch.float32, nb)
        _same_device(X, packed=packed, codebook16=codebook16, absmax=absmax)
    if absmax_code is not None and isinstance(offset, torch.Tensor):
        _buf(offset, "offset", torch.float32, 1)
        _same_device(X, offset=offset)
        name = "linear_4bit_nested_bf16_offptr"
        status = lib().linear_4bit_nested_bf16_offptr(_ptr(X), M, K, _ptr(packed), _ptr(codebook16),
                                                      _ptr(absmax_code), _ptr(qmap2), _ptr(absmax2), _ptr(offset),
                                                      N, blocksize, _ptr(out), _stream(X.device))
    elif absmax_code is not None:
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


def act_tables_k4(codebook16, tables=None):
    """Prepared assignment tables of a 16-entry codebook (uint8 tensor of
    kbit_act_tables_bytes() bytes), for ``quantize_act_fwht_k4_bf16(...,
    tables=...)``: built once instead of by every workgroup of every call."""
    torch = _torch()
    _buf(codebook16, "codebook16", torch.float32, 16)
    nbytes = lib().kbit_act_tables_bytes()
    if tables is None:
        tables = torch.empty(nbytes, dtype=torch.uint8, device=codebook16.device)
    _buf(tables, "tables", torch.uint8, nbytes)
    _same_device(codebook16, tables=tables)
    _check("act_tables_k4", lib().act_tables_k4(_ptr(codebook16), _ptr(tables), _stream(codebook16.device)))
    return tables


def quantize_act_fwht_k4_bf16(X, sign_bits, codebook16=None, row_norm=None, packed=None, perm=None, tables=None):
    """Token norm + sign flip + block FWHT (h = largest power of two dividing
    d) + Lloyd-Max assignment of bf16 [rows, d]; with ``perm`` (int32 [d])
    the columns are permuted first (quantize_act_rpbh_k4_bf16).  Give either
    ``codebook16`` or ``tables`` (from act_tables_k4)."""
    torch = _torch()
    if X.dtype != torch.bfloat16 or X.dim() != 2:
        raise TypeError("X must be a 2-D bfloat16 tensor")
    if (codebook16 is None) == (tables is None):
        raise TypeError("give exactly one of codebook16 and tables")
    rows, d = X.shape
    if row_norm is None:
        row_norm = torch.empty(rows, dtype=torch.float32, device=X.device)
    if packed is None:
        packed = torch.empty(n_words(rows * d, 4), dtype=torch.int32, device=X.device)
    _buf(sign_bits, "sign_bits", sign_bits.dtype if sign_bits.dtype in (torch.int32, torch.uint32) else torch.int32,
         -(-d // 32))
    if tables is None:
        _buf(codebook16, "codebook16", torch.float32, 16)
        cb, suffix = codebook16, ""
    else:
        _buf(tables, "tables", torch.uint8, lib().kbit_act_tables_bytes())
        cb, suffix = tables, "_tables"
    _buf(row_norm, "row_norm", torch.float32, rows)
    _buf(packed, "packed", torch.int32, n_words(rows * d, 4))
    _same_device(X, sign_bits=sign_bits, codebook16=cb, row_norm=row_norm, packed=packed, perm=perm)
    if perm is None:
        name = "quantize_act_fwht_k4_bf16" + suffix
        status = getattr(lib(), name)(_ptr(X), rows, d, _ptr(sign_bits), _ptr(cb), _ptr(row_norm), _ptr(packed),
                                      _stream(X.device))
    else:
        if perm.dtype != torch.int32 or perm.numel() != d:
            raise TypeError("perm must be an int32 tensor of d entries")
        name = "quantize_act_rpbh_k4_bf16" + suffix
        status = getattr(lib(), name)(_ptr(X), rows, d, _ptr(perm), _ptr(sign_bits), _ptr(cb), _ptr(row_norm),
                                      _ptr(packed), _stream(X.device))
    _check(name, status)
    return packed, row_norm


def quantize_act_rpbh_k4_bf16(X, perm, sign_bits, codebook16=None, row_norm=None, packed=None, tables=None):
    """Column permutation, then quantize_act_fwht_k4_bf16's path."""
    return quantize_act_fwht_k4_bf16(X, sign_bits, codebook16, row_norm=row_norm, packed=packed, perm=perm,
                                     tables=tables)


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
