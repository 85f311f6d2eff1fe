"""Exact-rational emulation of IEEE binary32 rounding, for pinning the oracle.

Independent of numpy's float32 arithmetic: every value is a Fraction and the
rounding to the nearest binary32 (ties to even) is done by integer
arithmetic here.
"""
from fractions import Fraction
import struct


def rnd32(q):
    """Round a Fraction to the nearest binary32 value (ties to even); returns Fraction."""
    q = Fraction(q)
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    # now 2^e <= a < 2^(e+1)
    e = max(e, -126)
    ulp = Fraction(2) ** (e - 23)
    m = a / ulp
    n = m.numerator // m.denominator
    rem = m - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * n * ulp


def f32_to_frac(x):
    return Fraction(float(x))


def frac_to_f32_bits(q):
    return struct.unpack("<I", struct.pack("<f", float(q)))[0]


def rnd_bf16(q):
    """Round a binary32-representable Fraction to bf16 (ties to even) -> Fraction."""
    q = Fraction(q)
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, -126)
    ulp = Fraction(2) ** (e - 7)
    m = a / ulp
    n = m.numerator // m.denominator
    rem = m - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * n * ulp


def rint_even(q):
    q = Fraction(q)
    n = q.numerator // q.denominator
    rem = q - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return n
