"""Blockwise absmax k-bit codebook quantize / pack / unpack / dequantize.

Test infrastructure only.  Follows [QLORA-2] PATCH 001,
``tests/test_kbit_quantization.py`` (``quantize_kbit_ref``,
``dequantize_kbit_ref``, ``pack_kbit_ref``, ``unpack_kbit_ref``) and the
production kernels ``kQuantizeBlockwise_kbit`` / ``kDequantizeBlockwise_kbit``
of ``csrc/kernels.cu``, generalised from blocksize 32 to any power-of-two
block size B (the nested-dequant PR [PR2051] Validation covers outer block
sizes 32 through 4096).

quantize (per block b of B consecutive elements; the last block may be short
and only its real elements count):
  1. x = exact fp32 widening of the element;
  2. a_b = max |x| over the block, returned unclamped;
  3. x_n = RN(x / max(a_b, 1e-8f))      (IEEE binary32 division);
  4. idx = the smallest i minimising |RN(x_n - c_i)|  (first index wins ties,
     as the kernel's strict "<" scan from i = 0 and torch.argmin both do).
pack: for each group g of 32 elements, K uint32 words; bit t of word
  g*K + j is bit j of idx[32g + t]; positions past n are 0.
dequantize: out_e = RN_T(RN(c[idx_e] * a_{floor(e/B)})).

Parity: pinned in ``tests/test_oracle_kbit.py`` (brute-force scalar search,
the printed K=3 pack pattern, round trips, error bounds, MSE/SQNR floors).
"""

import numpy as np

from .numerics import narrow

F32 = np.float32
ABSMAX_EPS = np.float32(1e-8)
GROUP = 32
_CHUNK = 1 << 20


def nearest_code(xn, codebook):
    """First-index argmin of |RN(x_n - c_i)| for float32 x_n (vectorised)."""
    xn = np.asarray(xn, dtype=np.float32).ravel()
    c = np.asarray(codebook, dtype=np.float32).ravel()
    out = np.empty(xn.size, dtype=np.uint8)
    for s in range(0, xn.size, _CHUNK):
        d = np.abs(xn[s:s + _CHUNK, None] - c[None, :])   # float32 ops
        out[s:s + _CHUNK] = np.argmin(d, axis=1)          # first minimum
    return out


def block_absmax(x, B):
    """Per-block max |x| (unclamped); the last block holds only real elements."""
    x = np.asarray(x, dtype=np.float32).ravel()
    n = x.size
    nb = -(-n // B)
    pad = nb * B - n
    ax = np.abs(x)
    if pad:
        ax = np.concatenate([ax, np.zeros(pad, np.float32)])  # |x| >= 0
    return ax.reshape(nb, B).max(axis=1) if nb else np.zeros(0, np.float32)


def normalize(x, absmax, B):
    """x_n = RN(x / max(a_b, 1e-8f)), one IEEE division per element."""
    x = np.asarray(x, dtype=np.float32).ravel()
    s = np.maximum(absmax, ABSMAX_EPS).astype(np.float32)
    blk = np.arange(x.size, dtype=np.int64) // B
    return (x / s[blk]).astype(np.float32)


def quantize(x, codebook, B):
    """Returns (idx uint8[n], absmax float32[ceil(n/B)])."""
    x = np.asarray(x, dtype=np.float32).ravel()
    a = block_absmax(x, B)
    idx = np.empty(x.size, dtype=np.uint8)
    for s in range(0, x.size, _CHUNK):
        e = min(x.size, s + _CHUNK)
        # chunk boundaries are multiples of B (B divides 2^20 for B <= 4096)
        xn = normalize(x[s:e], a[s // B:-(-e // B)], B)
        idx[s:e] = nearest_code(xn, codebook)
    return idx, a


def pack(idx, K):
    """Bit-plane packing: uint32[ceil(n/32) * K]."""
    idx = np.asarray(idx, dtype=np.uint8).ravel()
    n = idx.size
    ng = -(-n // GROUP)
    pad = np.zeros(ng * GROUP, dtype=np.uint64)
    pad[:n] = idx
    g = pad.reshape(ng, GROUP)
    weights = np.uint64(1) << np.arange(GROUP, dtype=np.uint64)
    words = np.empty((ng, K), dtype=np.uint32)
    for j in range(K):
        bits = (g >> np.uint64(j)) & np.uint64(1)
        words[:, j] = (bits * weights).sum(axis=1).astype(np.uint32)
    return words.ravel()


def unpack(words, K, n):
    """Inverse of ``pack`` trimmed to n elements: uint8[n]."""
    words = np.asarray(words, dtype=np.uint32).ravel()
    ng = -(-n // GROUP)
    w = words[: ng * K].reshape(ng, K).astype(np.uint64)
    t = np.arange(GROUP, dtype=np.uint64)
    idx = np.zeros((ng, GROUP), dtype=np.uint64)
    for j in range(K):
        idx |= ((w[:, j:j + 1] >> t[None, :]) & np.uint64(1)) << np.uint64(j)
    return idx.ravel()[:n].astype(np.uint8)


def dequantize_values(idx, scales, codebook, B):
    """fp32 values RN(c[idx_e] * scale_{e // B})."""
    idx = np.asarray(idx).ravel()
    c = np.asarray(codebook, dtype=np.float32)
    s = np.asarray(scales, dtype=np.float32)
    blk = np.arange(idx.size, dtype=np.int64) // B
    return (c[idx] * s[blk]).astype(np.float32)


def dequantize(idx, absmax, codebook, B, out_dtype):
    """out = RN_T(RN(c[idx] * absmax_block)); bf16 returned as raw uint16."""
    return narrow(dequantize_values(idx, absmax, codebook, B), out_dtype)


def quantize_packed(x, codebook, K, B):
    """quantize followed by pack: (words, absmax)."""
    idx, a = quantize(x, codebook, B)
    return pack(idx, K), a


def dequantize_packed(words, absmax, codebook, K, n, B, out_dtype):
    """unpack followed by dequantize."""
    return dequantize(unpack(words, K, n), absmax, codebook, B, out_dtype)
