"""Exact rational helpers for pinning the oracle (test-side, independent of oracle/).

Rounding of an exact rational to a binary floating-point format with p
significand bits (implicit bit included) and minimum normal exponent emin,
round to nearest, ties to even.  Overflow is not modelled (callers stay in range).
"""
from fractions import Fraction
import struct

F32 = (24, -126)
BF16 = (8, -126)


def round_to_format(fr: Fraction, p: int, emin: int) -> Fraction:
    fr = Fraction(fr)
    if fr == 0:
        return Fraction(0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    quantum = Fraction(2) ** (e - (p - 1))
    n = a / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * quantum


def f32(fr) -> Fraction:
    return round_to_format(Fraction(fr), *F32)


def bf16(fr) -> Fraction:
    return round_to_format(Fraction(fr), *BF16)


def rne_int(fr: Fraction) -> int:
    """Round a rational to the nearest integer, ties to even."""
    fr = Fraction(fr)
    fl = fr.numerator // fr.denominator
    rem = fr - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return fl


def bf16_bits_of(fr: Fraction) -> int:
    """Bits of a value that is exactly representable in bf16."""
    v = float(fr)
    b = struct.unpack("<I", struct.pack("<f", v))[0]
    assert b & 0xFFFF == 0, "value is not a bf16"
    return b >> 16


# All non-negative finite e4m3fn values by code (0x00..0x7E), from the format
# definition: exponent field e (bias 7), mantissa m; e == 0 is subnormal m * 2^-9.
def e4m3fn_value(code: int) -> Fraction:
    s = -1 if code & 0x80 else 1
    e = (code >> 3) & 0xF
    m = code & 7
    if e == 15 and m == 7:
        raise ValueError("NaN")
    if e == 0:
        return s * Fraction(m, 512)
    return s * (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)


E4M3_POS = [(c, e4m3fn_value(c)) for c in range(0x7F)]


def e4m3fn_nearest(fr: Fraction) -> int:
    """Brute force: nearest finite e4m3fn code, ties to the even code, saturating at 448."""
    fr = Fraction(fr)
    sign = 0x80 if fr < 0 else 0
    a = min(abs(fr), Fraction(448))
    best = None
    for c, v in E4M3_POS:
        d = abs(v - a)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1] | sign
