"""Exact-rational model of IEEE binary rounding, used to pin the oracle's
float32/float16 quantization arithmetic against arithmetic that is not numpy's.

Each operation is computed exactly with ``fractions.Fraction`` and then rounded
to the target format (nearest, ties to even, gradual underflow), which is what
IEEE 754 prescribes for +, -, *, / and for format conversion.
"""
from __future__ import annotations

from fractions import Fraction

# (significand bits incl. the implicit one, minimum normal exponent, maximum exponent)
F32 = (24, -126, 127)
F16 = (11, -14, 15)


def _floor_log2(a: Fraction) -> int:
    e = a.numerator.bit_length() - a.denominator.bit_length()
    # adjust so that 2**e <= a < 2**(e+1)
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def round_half_even_int(q: Fraction) -> int:
    n = q.numerator // q.denominator
    r = q - n
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return n


def round_fmt(x: Fraction, fmt) -> Fraction:
    mant, emin, emax = fmt
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = max(_floor_log2(a), emin)
    ulp = Fraction(2) ** (e - mant + 1)
    n = round_half_even_int(a / ulp)
    r = n * ulp
    if r >= Fraction(2) ** (emax + 1):
        raise OverflowError("overflow")
    return sign * r


def f32(x) -> Fraction:
    return round_fmt(Fraction(x), F32)


def f16(x) -> Fraction:
    return round_fmt(Fraction(x), F16)


def quantize_row_exact(xs, steps=254, lo=-128, hi=127):
    """The INT8 row contract (or, with steps=14, lo=-8, hi=7, the INT4 one),
    one IEEE operation at a time, in exact rationals.

    xs: iterable of exact values (bfloat16 values are exact float32 values).
    Returns (codes list[int], scale Fraction, zero Fraction)."""
    xs = [Fraction(x) for x in xs]
    mn, mx = min(xs), max(xs)
    z = f16(f32(f32(mx + mn) * Fraction(1, 2)))
    s = f16(f32(f32(mx - mn) / steps))
    if s == 0:
        s = Fraction(1)
    codes = []
    for x in xs:
        q = f32(f32(x - z) / s)
        codes.append(max(lo, min(hi, round_half_even_int(q))))
    return codes, s, z


def fp8_scale_exact(xs):
    """f16(f32(max|x| / 448)), 1 if that rounds to 0 (the FP8 row scale)."""
    amax = max(abs(Fraction(x)) for x in xs)
    s = f16(f32(amax / 448))
    return Fraction(1) if s == 0 else s
