"""Exact-rational IEEE rounding, written independently of numpy and of the
oracle, used to pin the oracle's rounding decisions.

Every value is a fractions.Fraction; rounding is done by exact integer
arithmetic, so a result here does not depend on any floating-point unit.
"""
from __future__ import annotations

import math
import struct
from fractions import Fraction


def _round_half_even_int(x: Fraction) -> int:
    fl = math.floor(x)
    rem = x - fl
    if rem > Fraction(1, 2):
        return fl + 1
    if rem < Fraction(1, 2):
        return fl
    return fl if fl % 2 == 0 else fl + 1


def rne_int(x: Fraction) -> int:
    """Round to the nearest integer, ties to even."""
    return _round_half_even_int(Fraction(x))


def round_binary(x: Fraction, mant_bits: int, emin: int, emax: int) -> Fraction:
    """Round x to the nearest value of a binary format with `mant_bits`
    explicit fraction bits, minimum normal exponent emin, max exponent emax
    (ties to even; overflow returns +-inf as float)."""
    x = Fraction(x)
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = math.floor(math.log2(a.numerator) - math.log2(a.denominator))
    # fix possible off-by-one of the float log
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    ulp = Fraction(2) ** (e - mant_bits)
    r = _round_half_even_int(a / ulp) * ulp
    if r >= Fraction(2) ** (emax + 1):
        return sign * float("inf")
    return sign * r


def rn32(x: Fraction) -> Fraction:
    return round_binary(x, 23, -126, 127)


def rn16(x: Fraction) -> Fraction:
    return round_binary(x, 10, -14, 15)


def f32_bits(x: Fraction) -> int:
    return struct.unpack("<I", struct.pack("<f", float(x)))[0]


def f32_from_bits(b: int) -> Fraction:
    return Fraction(struct.unpack("<f", struct.pack("<I", b))[0])


# OCP E4M3: enumerate the finite non-negative values from the format's fields
def e4m3_values():
    vals = []
    for e in range(16):
        for m in range(8):
            if e == 15 and m == 7:
                continue
            if e == 0:
                vals.append(Fraction(m, 8) * Fraction(2) ** (1 - 7))
            else:
                vals.append((1 + Fraction(m, 8)) * Fraction(2) ** (e - 7))
    return vals     # index = code (0..126)


def e4m3_round(x: Fraction) -> int:
    """Nearest E4M3 code by exhaustive search, ties to the even code,
    saturating at 448; sign bit kept."""
    vals = e4m3_values()
    a = abs(Fraction(x))
    best = None
    for c, v in enumerate(vals):
        dist = abs(a - v)
        if best is None or dist < best[0] or (dist == best[0] and c % 2 == 0):
            best = (dist, c)
    code = best[1]
    return code | (0x80 if x < 0 else 0)


def rn64(x: Fraction) -> Fraction:
    return round_binary(x, 52, -1022, 1023)
