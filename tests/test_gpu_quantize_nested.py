"""GPU parity: quantize straight to the nested 4-bit state in two kernels
(quantize_4bit_nested_*), whose quantize kernel also sums its own block
maxima for the mean offset.

Bar: bit-exact against the oracle run from the input alone
(``oracle.kbit.quantize_packed`` for the words and absmax, then
``oracle.nested.encode`` on the oracle's absmax for codes, absmax2 and the
offset).  The large cases repeat a seeded base array whole, so that their
expected words and absmax are the base's repeated (blocks and 32-groups line
up with the period) and the oracle runs on the base and the tail only; they
are sized so that each wave of the quantize kernel stages its block maxima
more than once (256 per round of the exact sums).
"""

import numpy as np
import pytest

import blockwise_bit_codebook_amd as kb
from blockwise_bit_codebook_amd import synth
from oracle import codebooks, kbit, nested, numerics
from tests.gpu_util import assert_bits_equal, bits, case, np_bits, to_dev

pytestmark = pytest.mark.gpu

DTYPES = ["fp32", "fp16", "bf16"]


def run(A, cb, q, B):
    import torch
    packed, absmax, code, a2, off = kb.quantize_4bit_nested(A, to_dev(cb), to_dev(q), B)
    torch.cuda.synchronize()
    return bits(packed), bits(absmax), bits(code), bits(a2), bits(off)[0]


def compare(got, ww, wa, q, what):
    words, absmax, code, a2, off = got
    assert_bits_equal(absmax, np_bits(wa), f"absmax {what}")
    assert_bits_equal(words, ww, f"words {what}")
    wc, wa2, woff = nested.encode(wa, q)
    assert off == np.float32(woff).view(np.uint32), (what, hex(off), hex(np.float32(woff).view(np.uint32)))
    assert_bits_equal(a2, np_bits(wa2), f"absmax2 {what}")
    assert_bits_equal(code, wc, f"codes {what}")


def check(x, dtype, B, what, cb=None, q=None):
    cb = codebooks.nf(4) if cb is None else cb
    q = codebooks.dynamic_map8() if q is None else q
    case(f"quantize to nested state {what} dtype={dtype} B={B} n={x.size}")
    got = run(to_dev(x, dtype), cb, q, B)
    ww, wa = kbit.quantize_packed(numerics.widen(x, dtype), cb, 4, B)
    compare(got, ww, wa, q, what)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("B", [32, 64, 256, 1024, 4096])
def test_sizes(dtype, B):
    for n in (1, 31, 64, 513, 4097, 65613, 3 * 4096 * 8 + 1000):
        x = synth.normal(n, seed=2000 + n + B, dtype=dtype)
        check(x, dtype, B, f"n={n}")


@pytest.mark.parametrize("dtype", DTYPES)
def test_same_as_the_two_calls(dtype):
    # the plain quantize followed by the encoder gives the same bits
    import torch
    n, B = 1_000_003, 64
    x = synth.normal(n, seed=77, dtype=dtype)
    cb, q = codebooks.fp4(), codebooks.dynamic_map8()
    case(f"quantize to nested state vs the two calls dtype={dtype} n={n}")
    A = to_dev(x, dtype)
    got = run(A, cb, q, B)
    packed, absmax = kb.quantize_kbit(A, to_dev(cb), 4, B)
    code, a2, off = kb.quantize_nested_absmax(absmax, to_dev(q))
    torch.cuda.synchronize()
    for g, w, what in zip(got, (bits(packed), bits(absmax), bits(code), bits(a2), bits(off)[0]),
                          ("words", "absmax", "codes", "absmax2", "offset")):
        assert_bits_equal(np.asarray(g), np.asarray(w), what)


def test_special_blocks():
    # fp32 input whose block maxima span many binades (each wave's exact sums
    # take values far below its top through the exponent bins), plus blocks
    # with an infinity, a NaN, zeros and subnormal maxima
    rng = np.random.default_rng(5)
    B = 64
    nb = 40000
    x = synth.normal(nb * B, seed=6, dtype="fp32").reshape(nb, B)
    scale = np.ldexp(np.float32(1.0), rng.integers(-140, 100, nb)).astype(np.float32)
    x = (x * scale[:, None]).astype(np.float32)
    x[7] = 0.0
    x[9, :] = np.float32(1e-44)
    base = x.reshape(-1).copy()
    check(base, "fp32", B, "wide binades")
    for name, (blk, val) in {"inf": (1234, np.inf), "neg inf": (20000, -np.inf), "nan": (333, np.nan)}.items():
        y = x.copy()
        y[blk, 5] = val
        check(y.reshape(-1), "fp32", B, name)


@pytest.mark.parametrize("dtype,B,logn,reps,tail", [
    ("bf16", 64, 25, 8, 4099),          # 64 rows of 512 per wave: the stage fills twice
    ("fp16", 32, 25, 2, 77),            # 16 rows per wave, 16 maxima per row: one full stage
    ("fp32", 32, 25, 4, 1000),          # two-row ring, 32 rows per wave: two full stages
    ("bf16", 1024, 25, 65, 1025 * 700 + 3),  # about 260 blocks of 1024 per wave
])
def test_stage_fills(dtype, B, logn, reps, tail):
    import torch
    base = synth.normal(1 << logn, seed=900 + B, dtype=dtype)
    cb, q = codebooks.nf(4), codebooks.dynamic_map8()
    n = reps * base.size + tail
    case(f"quantize to nested state, repeated base dtype={dtype} B={B} n={n}")
    A = torch.cat([to_dev(base, dtype).repeat(reps), to_dev(base[:tail], dtype)])
    got = run(A, cb, q, B)
    del A
    torch.cuda.empty_cache()
    x32 = numerics.widen(base, dtype)
    ww, wa = kbit.quantize_packed(x32, cb, 4, B)
    tw, ta = kbit.quantize_packed(x32[:tail], cb, 4, B)
    compare(got, np.concatenate([np.tile(ww, reps), tw]), np.concatenate([np.tile(wa, reps), ta]), q,
            f"{reps} x 2^{logn} + {tail}")
