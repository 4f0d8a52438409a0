"""Exact-rational model of binary32 arithmetic, used to pin the oracle.

Written from IEEE 754-2019 (round to nearest, ties to even; gradual
underflow) and the flush rule of the Open-1B report §2.1 "Subnormals"
(a subnormal result or input becomes a zero of the same sign).  It shares
nothing with the C oracle: values are Python Fractions, rounding is done by
integer arithmetic on the exact quotient.
"""
from fractions import Fraction
import math
import struct

EMIN = -126          # smallest normal exponent
P = 24               # significand bits


def bits_to_float(b: int) -> float:
    return struct.unpack("<f", struct.pack("<I", b & 0xFFFFFFFF))[0]


def float_to_bits(f: float) -> int:
    return struct.unpack("<I", struct.pack("<f", f))[0]


def round_binary32(x: Fraction) -> Fraction:
    """Round an exact rational to binary32 (RNE, gradual underflow, no
    overflow handling: callers stay in range)."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = math.floor(math.log2(a.numerator) - math.log2(a.denominator))
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    q = max(e, EMIN) - (P - 1)            # quantum of the result's binade
    m = a / (Fraction(2) ** q)
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * Fraction(fl) * (Fraction(2) ** q)


def is_subnormal(x: Fraction) -> bool:
    return x != 0 and abs(x) < Fraction(2) ** EMIN


def op(x: Fraction) -> Fraction:
    """One binary32 operation's result: round, then flush a subnormal."""
    r = round_binary32(x)
    return Fraction(0) if is_subnormal(r) else r


def to_float(x: Fraction) -> float:
    return float(x)
