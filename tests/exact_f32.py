"""Exact binary32 arithmetic from rational numbers, independent of numpy.

Used by the oracle's pins: each operation is evaluated exactly as a Fraction and
then rounded to the nearest binary32 value, ties to even (IEEE 754 default).
"""
from fractions import Fraction
import math
import struct

F32_MAX = (2 - Fraction(1, 2 ** 23)) * Fraction(2) ** 127
HALF_ULP_MAX = Fraction(2) ** 103  # half the spacing at the top binade


def bits_to_float(bits):
    return struct.unpack("<f", struct.pack("<I", bits & 0xFFFFFFFF))[0]


def float_to_bits(x):
    return struct.unpack("<I", struct.pack("<f", x))[0]


def round_f32(q, zero_sign=1.0):
    """Nearest binary32 to the rational q (ties to even), as a Python float."""
    q = Fraction(q)
    if q == 0:
        return 0.0 if zero_sign > 0 else -0.0
    sign = -1.0 if q < 0 else 1.0
    a = abs(q)
    if a >= F32_MAX + HALF_ULP_MAX:
        return sign * float("inf")
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    ulp = Fraction(2) ** (e - 23)
    n = a / ulp
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * float(fl * ulp)


def _neg(x):
    return math.copysign(1.0, x) < 0


def f32_div(a, b):
    return round_f32(Fraction(a) / Fraction(b), zero_sign=(-1.0 if _neg(a) != _neg(b) else 1.0))


def f32_mul(a, b):
    return round_f32(Fraction(a) * Fraction(b), zero_sign=(-1.0 if _neg(a) != _neg(b) else 1.0))


def f32_add(a, b):
    # an exact zero sum is +0 except (-0) + (-0) = -0
    return round_f32(Fraction(a) + Fraction(b), zero_sign=(-1.0 if _neg(a) and _neg(b) else 1.0))


def f32_sub(a, b):
    return f32_add(a, -b)
