"""Exact-arithmetic helpers for the oracle pins (pure Python, no numpy arithmetic).

These are written independently of the oracle: rounding a rational to binary32 or
binary16 is done here by explicit bit arithmetic on Fractions, not by numpy casts.
"""
from __future__ import annotations

import math
import struct
from fractions import Fraction


def round_to_format(x: Fraction, mant_bits: int, emin: int, emax: int) -> float:
    """Round the rational x to the nearest binary float with ``mant_bits`` significand
    bits (including the hidden bit), minimum normal exponent ``emin`` and maximum
    exponent ``emax``; ties to even; overflow to +-inf; subnormals kept."""
    if x == 0:
        return 0.0
    sign = -1 if x < 0 else 1
    a = abs(x)
    # exponent e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    ulp = Fraction(2) ** (e - (mant_bits - 1))
    q = a / ulp
    n = q.numerator // q.denominator
    r = q - n
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and n % 2 == 1):
        n += 1
    v = n * ulp
    if v >= Fraction(2) ** (emax + 1):
        return sign * math.inf
    return sign * float(v)


def f32(x: Fraction) -> float:
    return round_to_format(Fraction(x), 24, -126, 127)


def f16(x: Fraction) -> float:
    return round_to_format(Fraction(x), 11, -14, 15)


def f16_bits(v: float) -> int:
    """binary16 bit pattern of a float that is exactly representable in binary16."""
    return struct.unpack("<H", struct.pack("<e", v))[0]


def f32_bits(v: float) -> int:
    return struct.unpack("<I", struct.pack("<f", v))[0]


def f32_ulp(v: float) -> float:
    """Spacing of binary32 numbers at |v|."""
    if v == 0:
        return 2.0 ** -149
    e = math.frexp(abs(v))[1] - 1
    return 2.0 ** max(e - 23, -149)
