"""Exact rational arithmetic used to pin the oracle (test helper).

Binary32, bf16 and binary16 rounding are written out here from their definition
(nearest representable value, ties to the even significand, subnormals kept),
on Python Fractions. Nothing here calls the C oracle or the hardware's float
unit, so a slip in either (a contracted or double-precision division, a
reciprocal multiply, flush-to-zero, truncation instead of rounding) shows up as
a mismatch.
"""
from fractions import Fraction


def _floor_log2(a: Fraction) -> int:
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def round_to_format(v: Fraction, frac_bits: int, emin: int = -126) -> Fraction:
    """Nearest value with `frac_bits` stored fraction bits, exponent >= emin, ties to even."""
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = max(_floor_log2(a), emin)
    quantum = Fraction(2) ** (e - frac_bits)
    return sign * round(a / quantum) * quantum   # Fraction.__round__ is half-to-even


def f32(v: Fraction) -> Fraction:
    return round_to_format(v, 23)


def bf16(v: Fraction) -> Fraction:
    return round_to_format(v, 7)


def f16(v: Fraction) -> Fraction:
    """IEEE binary16: 10 stored fraction bits, exponents from -14 (subnormals below).
    Values rounding to 2^16 or beyond overflow (returned as None)."""
    r = round_to_format(v, 10, emin=-14)
    return None if abs(r) >= 2 ** 16 else r


def quantize_row(xs):
    """The absmax/127 rule on a row of exact values: (scale, [q])."""
    absmax = max((abs(x) for x in xs), default=Fraction(0))
    s = f32(absmax / 127)
    if s == 0:
        return s, [0] * len(xs)
    return s, [max(-127, min(127, round(f32(x / s)))) for x in xs]
