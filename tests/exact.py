"""Exact rational arithmetic for pinning the oracle (test helper, no numpy/C).

IEEE binary32 operations are defined as the exact result rounded to the
nearest representable value, ties to even.  These helpers compute that
definition with Python fractions so that tests can check the oracle against
the definition itself rather than against another floating-point library.
"""
from __future__ import annotations

import math
import struct
from fractions import Fraction

HALF = Fraction(1, 2)


def f32_bits(x: float) -> int:
    return struct.unpack("<I", struct.pack("<f", x))[0]


def bits_f32(b: int) -> float:
    return struct.unpack("<f", struct.pack("<I", b))[0]


def _floor_log2(a: Fraction) -> int:
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def round_half_even(q: Fraction) -> int:
    fl = math.floor(q)
    rem = q - fl
    if rem > HALF or (rem == HALF and fl % 2 == 1):
        fl += 1
    return fl


def rn32(v) -> float:
    """binary32 value nearest the rational v (ties to even), as a Python float."""
    v = Fraction(v)
    if v == 0:
        return 0.0
    sign = -1.0 if v < 0 else 1.0
    a = abs(v)
    lsb = max(_floor_log2(a) - 23, -149)
    step = Fraction(2) ** lsb
    r = round_half_even(a / step) * step
    if r >= Fraction(2) ** 128:
        return sign * math.inf
    return sign * float(r)


def rn_bf16_bits(v) -> int:
    """bfloat16 bit pattern nearest the rational v (ties to even)."""
    v = Fraction(v)
    if v == 0:
        return 0
    sign = 0x8000 if v < 0 else 0
    a = abs(v)
    lsb = max(_floor_log2(a) - 7, -133)
    step = Fraction(2) ** lsb
    r = round_half_even(a / step) * step
    if r >= Fraction(2) ** 128:
        return sign | 0x7F80
    return sign | (f32_bits(float(r)) >> 16)


def div32(x: float, s: float) -> float:
    return rn32(Fraction(x) / Fraction(s))


def quant_code(x: float, s: float) -> int:
    """clamp(rint(RN32(x / s)), -127, 127) from the definitions."""
    c = round_half_even(Fraction(div32(x, s)))
    return max(-127, min(127, c))


def scale_of(amax: float) -> float:
    """RN32(max(amax, RN32(1e-12)) / 127)."""
    guard = rn32(Fraction(1, 10**12))
    return div32(max(amax, guard), 127.0)
