"""Exact-arithmetic helpers for pinning the oracle.

Rounding of an exact rational to a binary floating-point format, written from
the IEEE 754 definition (round to nearest, ties to even) with Python's
``fractions.Fraction`` -- independent of any C or numpy float operation, so
that a test built on it checks the oracle's fp32/bf16 arithmetic rather than
re-running it.
"""
from __future__ import annotations

import math
import struct
from fractions import Fraction


def _round_half_even_int(r: Fraction) -> int:
    fl = math.floor(r)
    d = r - fl
    if d > Fraction(1, 2):
        return fl + 1
    if d < Fraction(1, 2):
        return fl
    return fl if fl % 2 == 0 else fl + 1


def round_to_format(r: Fraction, p: int, emin: int, emax: int) -> Fraction:
    """Nearest value of a binary format with p significant bits (ties even).

    emin/emax are the exponents of the smallest/largest normal binade
    (fp32: p=24, emin=-126, emax=127; bf16: p=8, same exponents).  Subnormals
    are handled (quantum 2**(emin-p+1)); overflow returns +-inf as a float.
    """
    if r == 0:
        return Fraction(0)
    sign = -1 if r < 0 else 1
    a = -r if r < 0 else r
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    q = Fraction(2) ** (e - p + 1)
    n = _round_half_even_int(a / q)
    v = n * q
    if v >= Fraction(2) ** (emax + 1):
        return Fraction(sign) * Fraction(10) ** 400  # stands for inf
    return sign * v


def fp32(r: Fraction) -> Fraction:
    return round_to_format(r, 24, -126, 127)


def bf16(r: Fraction) -> Fraction:
    return round_to_format(r, 8, -126, 127)


def f32_value(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", bits & 0xFFFFFFFF))[0]


def bf16_bits_value(bits: int) -> Fraction:
    return Fraction(f32_value((bits & 0xFFFF) << 16))


def bf16_bits_of(v: Fraction) -> int:
    """bf16 bit pattern of a value already representable in bf16."""
    f = float(v)
    u = struct.unpack("<I", struct.pack("<f", f))[0]
    assert u & 0xFFFF == 0, "value not representable in bf16"
    return u >> 16


def _fp32_neighbors(v: Fraction):
    """The fp32 values just below and above a positive fp32 value v."""
    f = float(v)
    u = struct.unpack("<I", struct.pack("<f", f))[0]
    lo = Fraction(struct.unpack("<f", struct.pack("<I", u - 1))[0])
    hi = Fraction(struct.unpack("<f", struct.pack("<I", u + 1))[0])
    return lo, hi


def sqrt_fp32(r: Fraction) -> Fraction:
    """Correctly rounded fp32 square root of a positive rational: the fp32
    value nearest to sqrt(r) (ties to even), decided by exact comparisons of
    squares against r (no floating-point square root is trusted)."""
    assert r > 0
    c = fp32(Fraction(math.sqrt(float(r))))  # estimate, then correct exactly
    while c * c > r:
        c = _fp32_neighbors(c)[0]
    while True:
        d = _fp32_neighbors(c)[1]
        if d * d <= r:
            c = d
        else:
            break
    # now c <= sqrt(r) < d: round by the midpoint
    m = (c + d) / 2
    if r < m * m:
        return c
    if r > m * m:
        return d
    even = (struct.unpack("<I", struct.pack("<f", float(c)))[0] & 1) == 0
    return c if even else d


def e4m3(r: Fraction) -> Fraction:
    """Nearest E4M3 value (4 significant bits, normal exponents -6 .. 8,
    subnormal quantum 2**-9; ties to even), magnitudes beyond the largest
    finite value 448 saturating to it."""
    v = round_to_format(r, 4, -6, 8)
    if abs(v) > 448:
        return Fraction(448) if v > 0 else Fraction(-448)
    return v


def f16(r: Fraction) -> Fraction:
    """Nearest IEEE binary16 value (11 significant bits, normal exponents
    -14 .. 15, ties to even); beyond the largest finite value rounds to the
    infinity stand-in of round_to_format."""
    return round_to_format(r, 11, -14, 15)
