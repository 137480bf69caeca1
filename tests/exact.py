"""Exact rational arithmetic used to pin the oracle.

These helpers never use the machine's floating point: values are Python
``Fraction`` objects and every IEEE rounding is carried out by counting units
in the last place.  They give an independent check of the C oracle, which uses
the host's fp32/fp64 hardware.
"""
from __future__ import annotations

from fractions import Fraction
import struct


def frac(x) -> Fraction:
    """Exact value of a Python float / numpy scalar."""
    return Fraction(float(x))


def _floor_log2(a: Fraction) -> int:
    """floor(log2(a)) for a > 0."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    # now 2^(e-1) < a < 2^(e+1); fix up
    if a >= Fraction(2) ** e:
        return e
    return e - 1


def round_binary(a: Fraction, mant_bits: int, min_exp: int) -> Fraction:
    """Round ``a`` to the nearest binary float with ``mant_bits`` significant bits (ties to even).

    ``min_exp`` is the exponent of the smallest subnormal unit (2**min_exp).
    Overflow is not modelled (inputs here are far from it).
    """
    if a == 0:
        return Fraction(0)
    sign = -1 if a < 0 else 1
    a = abs(a)
    e = _floor_log2(a)
    qexp = max(e - (mant_bits - 1), min_exp)
    unit = Fraction(2) ** qexp
    n = round(a / unit)  # Fraction.__round__ rounds half to even
    return sign * n * unit


def fl32(a: Fraction) -> Fraction:
    """IEEE binary32 round-to-nearest-even of an exact rational."""
    return round_binary(a, 24, -149)


def fl_bf16(a: Fraction) -> Fraction:
    """bfloat16 round-to-nearest-even of an exact rational."""
    return round_binary(a, 8, -133)


def rne_int(a: Fraction) -> int:
    """Round to the nearest integer, ties to even."""
    return int(round(a))


def bf16_bits(v: Fraction) -> int:
    """Bit pattern of a value exactly representable in bfloat16."""
    f = float(v)
    u = struct.unpack("<I", struct.pack("<f", f))[0]
    assert (u & 0xFFFF) == 0, "value is not a bfloat16"
    return u >> 16


def bf16_value(bits: int) -> Fraction:
    u = (int(bits) & 0xFFFF) << 16
    return Fraction(struct.unpack("<f", struct.pack("<I", u))[0])


def ulp_bf16(a: Fraction) -> Fraction:
    """Spacing of bfloat16 numbers at |a| (the unit of the binade containing a)."""
    if a == 0:
        return Fraction(2) ** -133
    e = _floor_log2(abs(a))
    return Fraction(2) ** max(e - 7, -133)
