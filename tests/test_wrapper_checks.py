"""Host-side checks of the Python binding's argument validation.

The C ABI takes raw pointers and cannot see sizes or element types, so the
binding checks every buffer before it passes an address on.  These tests
use CPU tensors: a bad buffer must raise an error that names it, and a
call whose buffers are all well formed gets as far as the placement check
("must live on the GPU") without reaching the library.
"""

import pytest

kb = pytest.importorskip("blockwise_bit_codebook_amd")
torch = pytest.importorskip("torch")

f32, u8, i32, bf16 = torch.float32, torch.uint8, torch.int32, torch.bfloat16


def z(n, dt):
    return torch.zeros(n, dtype=dt)


def placement_only(fn, *a, **kw):
    with pytest.raises(ValueError, match="must live on the GPU"):
        fn(*a, **kw)


def bad(exc, match, fn, *a, **kw):
    with pytest.raises(exc, match=match):
        fn(*a, **kw)


N, B, K = 1000, 64, 4
NB = -(-N // B)
NW = -(-N // 32) * K


def test_quantize_kbit():
    A = z(N, bf16)
    placement_only(kb.quantize_kbit, A, z(16, f32), K, B, absmax=z(NB, f32), packed=z(NW, i32))
    bad(ValueError, "codebook", kb.quantize_kbit, A, z(15, f32), K, B)
    bad(TypeError, "codebook", kb.quantize_kbit, A, z(16, torch.float64), K, B)
    bad(TypeError, "absmax", kb.quantize_kbit, A, z(16, f32), K, B, absmax=z(NB, u8))
    bad(ValueError, "absmax", kb.quantize_kbit, A, z(16, f32), K, B, absmax=z(NB - 1, f32))
    bad(TypeError, "absmax", kb.quantize_kbit, A, z(16, f32), K, B, absmax=z(NB, f32), absmax_format="e4m4")
    bad(ValueError, "packed", kb.quantize_kbit, A, z(16, f32), K, B, packed=z(NW - 1, i32))
    bad(TypeError, "packed", kb.quantize_kbit, A, z(16, f32), K, B, packed=z(NW, torch.int64))
    bad(ValueError, "k must be", kb.quantize_kbit, A, z(64, f32), 6, B)
    bad(ValueError, "blocksize", kb.quantize_kbit, A, z(16, f32), K, 0)
    bad(TypeError, "element dtype", kb.quantize_kbit, z(N, torch.float64), z(16, f32), K, B)


def test_dequantize_kbit():
    placement_only(kb.dequantize_kbit, z(NW, i32), z(16, f32), z(NB, f32), K, N, bf16, B)
    placement_only(kb.dequantize_kbit, z(NW, i32), z(16, f32), z(NB, u8), K, N, bf16, B)
    bad(ValueError, "packed", kb.dequantize_kbit, z(NW - 1, i32), z(16, f32), z(NB, f32), K, N, bf16, B)
    bad(ValueError, "codebook", kb.dequantize_kbit, z(NW, i32), z(8, f32), z(NB, f32), K, N, bf16, B)
    bad(ValueError, "absmax", kb.dequantize_kbit, z(NW, i32), z(16, f32), z(NB - 1, u8), K, N, bf16, B)
    bad(TypeError, "block scales", kb.dequantize_kbit, z(NW, i32), z(16, f32), z(NB, f32).half(), K, N, bf16, B)
    bad(TypeError, "out", kb.dequantize_kbit, z(NW, i32), z(16, f32), z(NB, f32), K, N, bf16, B,
        out=z(N, torch.float16))
    bad(ValueError, "out", kb.dequantize_kbit, z(NW, i32), z(16, f32), z(NB, f32), K, N, bf16, B, out=z(N - 1, bf16))
    bad(ValueError, "n must be", kb.dequantize_kbit, z(NW, i32), z(16, f32), z(NB, f32), K, -1, bf16, B)


def test_dequantize_4bit_nested():
    args = [z(-(-N // 32) * 4, i32), z(16, f32), z(NB, u8), z(256, f32), z(1, f32), 0.0, N, bf16, B]
    placement_only(kb.dequantize_4bit_nested, *args)
    for i, (t, what, exc) in enumerate([(z(10, i32), "packed", ValueError), (z(15, f32), "codebook16", ValueError),
                                        (z(NB - 1, u8), "absmax_code", ValueError),
                                        (z(NB, f32), "absmax_code", TypeError),
                                        (z(255, f32), "qmap2", ValueError), (z(0, f32), "absmax2", ValueError)]):
        a = list(args)
        a[{"packed": 0, "codebook16": 1, "absmax_code": 2, "qmap2": 3, "absmax2": 4}[what]] = t
        bad(exc, what, kb.dequantize_4bit_nested, *a)
    bad(ValueError, "out", kb.dequantize_4bit_nested, *args, out=z(N - 1, bf16))


def test_nested_encode():
    nb = 1000
    a = z(nb, f32)
    placement_only(kb.quantize_nested_absmax, a, z(256, f32))
    placement_only(kb.quantize_nested_absmax_noalloc, a, z(256, f32), z(nb, u8), z(4, f32), z(1, f32))
    bad(ValueError, "qmap2", kb.quantize_nested_absmax, a, z(255, f32))
    bad(TypeError, "absmax", kb.quantize_nested_absmax, z(nb, torch.float16), z(256, f32))
    bad(ValueError, "absmax_code", kb.quantize_nested_absmax, a, z(256, f32), absmax_code=z(nb - 1, u8))
    bad(ValueError, "absmax2", kb.quantize_nested_absmax, a, z(256, f32), absmax2=z(3, f32))
    bad(TypeError, "offset", kb.quantize_nested_absmax, a, z(256, f32), offset=z(1, torch.float64))
    bad(ValueError, "workspace", kb.quantize_nested_absmax, a, z(256, f32), workspace=z(8, u8))
    bad(ValueError, "absmax2", kb.quantize_nested_absmax_noalloc, a, z(256, f32), z(nb, u8), z(3, f32), z(1, f32))
    bad(ValueError, "offset", kb.quantize_nested_absmax_noalloc, a, z(256, f32), z(nb, u8), z(4, f32), z(0, f32))


def test_quantize_4bit_nested():
    A, q = z(N, bf16), z(256, f32)
    placement_only(kb.quantize_4bit_nested, A, z(16, f32), q, B)
    bad(ValueError, "codebook16", kb.quantize_4bit_nested, A, z(8, f32), q, B)
    bad(ValueError, "qmap2", kb.quantize_4bit_nested, A, z(16, f32), z(255, f32), B)
    bad(ValueError, "absmax", kb.quantize_4bit_nested, A, z(16, f32), q, B, absmax=z(NB - 1, f32))
    bad(TypeError, "packed", kb.quantize_4bit_nested, A, z(16, f32), q, B, packed=z(NW, f32))
    bad(ValueError, "absmax_code", kb.quantize_4bit_nested, A, z(16, f32), q, B, absmax_code=z(NB - 1, u8))
    bad(ValueError, "workspace", kb.quantize_4bit_nested, A, z(16, f32), q, B, workspace=z(8, u8))
    bad(TypeError, "element", kb.quantize_4bit_nested, z(N, torch.int16), z(16, f32), q, B)


def test_linear_4bit():
    M, Kd, Nn = 4, 128, 64
    X = z(M * Kd, bf16).view(M, Kd)
    nb = Nn * Kd // B
    pw = Nn * Kd // 32 * 4
    placement_only(kb.linear_4bit, X, z(pw, i32), z(16, f32), Nn, B, absmax=z(nb, f32))
    placement_only(kb.linear_4bit, X, z(pw, i32), z(16, f32), Nn, B, absmax_code=z(nb, u8), qmap2=z(256, f32),
                   absmax2=z(1, f32), offset=0.0)
    bad(ValueError, "packed", kb.linear_4bit, X, z(pw - 1, i32), z(16, f32), Nn, B, absmax=z(nb, f32))
    bad(ValueError, "absmax", kb.linear_4bit, X, z(pw, i32), z(16, f32), Nn, B, absmax=z(nb - 1, f32))
    bad(ValueError, "qmap2", kb.linear_4bit, X, z(pw, i32), z(16, f32), Nn, B, absmax_code=z(nb, u8),
        qmap2=z(16, f32), absmax2=z(1, f32), offset=0.0)
    bad(ValueError, "out", kb.linear_4bit, X, z(pw, i32), z(16, f32), Nn, B, absmax=z(nb, f32),
        out=z(M * Nn - 1, bf16))


def test_activation_path():
    rows, d = 4, 512
    X = z(rows * d, bf16).view(rows, d)
    placement_only(kb.quantize_act_fwht_k4_bf16, X, z(d // 32, i32), z(16, f32))
    bad(ValueError, "sign_bits", kb.quantize_act_fwht_k4_bf16, X, z(d // 32 - 1, i32), z(16, f32))
    bad(TypeError, "sign_bits", kb.quantize_act_fwht_k4_bf16, X, z(d // 32, f32), z(16, f32))
    bad(ValueError, "codebook16", kb.quantize_act_fwht_k4_bf16, X, z(d // 32, i32), z(15, f32))
    bad(ValueError, "row_norm", kb.quantize_act_fwht_k4_bf16, X, z(d // 32, i32), z(16, f32), row_norm=z(3, f32))
    bad(ValueError, "packed", kb.quantize_act_fwht_k4_bf16, X, z(d // 32, i32), z(16, f32), packed=z(10, i32))
    bad(TypeError, "perm", kb.quantize_act_rpbh_k4_bf16, X, z(d, torch.int64), z(d // 32, i32), z(16, f32))


def test_activation_prepared_tables():
    rows, d = 4, 512
    X = z(rows * d, bf16).view(rows, d)
    tb = kb.lib().kbit_act_tables_bytes()
    placement_only(kb.quantize_act_fwht_k4_bf16, X, z(d // 32, i32), tables=z(tb, u8))
    placement_only(kb.act_tables_k4, z(16, f32))
    bad(ValueError, "tables", kb.quantize_act_fwht_k4_bf16, X, z(d // 32, i32), tables=z(tb - 1, u8))
    bad(TypeError, "tables", kb.quantize_act_fwht_k4_bf16, X, z(d // 32, i32), tables=z(tb, f32))
    bad(TypeError, "exactly one", kb.quantize_act_fwht_k4_bf16, X, z(d // 32, i32))
    bad(TypeError, "exactly one", kb.quantize_act_fwht_k4_bf16, X, z(d // 32, i32), z(16, f32), tables=z(tb, u8))
    bad(ValueError, "codebook16", kb.act_tables_k4, z(15, f32))
    bad(ValueError, "tables", kb.act_tables_k4, z(16, f32), tables=z(tb - 1, u8))
