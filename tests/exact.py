"""Exact rational reference arithmetic for pinning the oracle.

Independent of numpy's float arithmetic: every value is a Python
``fractions.Fraction`` and rounding to a binary format is done here from its
definition (round to nearest, ties to even, gradual underflow, overflow to
infinity).
"""

from fractions import Fraction
import math
import struct

# (significand bits including the implicit one, minimum normal exponent, maximum exponent)
FP32 = (24, -126, 127)
FP16 = (11, -14, 15)
BF16 = (8, -126, 127)


def frac(x):
    """Exact value of a finite binary float (Python float / numpy scalar)."""
    return Fraction(float(x))


def _floor_log2(a):
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if a < Fraction(2) ** e:
        e -= 1
    elif a >= Fraction(2) ** (e + 1):
        e += 1
    return e


def round_to(q, fmt):
    """Round an exact rational to the format: returns a Fraction or +-inf."""
    p, emin, emax = fmt
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = max(_floor_log2(a), emin)
    quantum = Fraction(2) ** (e - (p - 1))
    m = a / quantum
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * quantum
    if r >= Fraction(2) ** (emax + 1):
        return sign * math.inf
    return sign * r


def f32(q):
    """Round to binary32 and return a Python float holding that value."""
    r = round_to(q, FP32)
    return float(r)


def f32_bits(x):
    return struct.unpack("<I", struct.pack("<f", float(x)))[0]


def nearest_first(xn, codebook):
    """Strict-< scan from index 0 of |RN32(x_n - c_i)| with exact arithmetic."""
    best, bestd = 0, None
    for i, c in enumerate(codebook):
        d = abs(Fraction(f32(frac(xn) - frac(c))))
        if bestd is None or d < bestd:
            best, bestd = i, d
    return best
