"""Exact-arithmetic evaluation of single rounding steps, for pinning the oracle.

Written independently of ``oracle/``: values are Python ``Fraction`` objects,
every operation is exact, and a result is rounded to FP32 or BF16 only where
the tail's formulas round, by round-to-nearest-even written from the IEEE 754
definition (the quantum of a binade, the quotient rounded half to even).  A
reciprocal square root is correctly rounded from an integer square root
carried 160 bits past the result.

These evaluations are slow (pure Python) and meant for a few hundred values.
A golden value or an oracle step checked against them is fixed by the
mathematics, not by another floating-point implementation.
"""
from __future__ import annotations

import math
import struct
from fractions import Fraction

FP32 = (24, -126)  # significant bits, smallest normal exponent
BF16 = (8, -126)


def _floor_log2(x: Fraction) -> int:
    """e with 2^e <= x < 2^(e+1), for x > 0."""
    e = x.numerator.bit_length() - x.denominator.bit_length()
    if Fraction(2) ** e > x:
        e -= 1
    elif Fraction(2) ** (e + 1) <= x:
        e += 1
    return e


def rne(x: Fraction, fmt=FP32) -> Fraction:
    """The nearest value of the format to x, ties to the even significand
    (no overflow handling: the callers stay far inside the range)."""
    if x == 0:
        return Fraction(0)
    p, emin = fmt
    sign = -1 if x < 0 else 1
    a = -x if x < 0 else x
    e = max(_floor_log2(a), emin)
    quantum = Fraction(2) ** (e - (p - 1))
    q = a / quantum
    n = math.floor(q)
    rest = q - n
    if rest > Fraction(1, 2) or (rest == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * n * quantum


def f32_value(bits: int) -> Fraction:
    """The exact value of an FP32 bit pattern (finite)."""
    f = struct.unpack("<f", struct.pack("<I", bits & 0xFFFFFFFF))[0]
    return Fraction(f)


def f32_bits(x: Fraction) -> int:
    """The bit pattern of an FP32 value x (x must already be an FP32 value)."""
    f = float(x)
    b = struct.unpack("<I", struct.pack("<f", f))[0]
    assert Fraction(struct.unpack("<f", struct.pack("<I", b))[0]) == x, "not an FP32 value"
    return b


def bf16_value(bits: int) -> Fraction:
    return f32_value((bits & 0xFFFF) << 16)


def bf16_bits(x: Fraction) -> int:
    """The BF16 bit pattern of a BF16 value x."""
    b = f32_bits(x)
    assert b & 0xFFFF == 0, "not a BF16 value"
    return b >> 16


def mul(a, b, fmt=FP32):
    return rne(Fraction(a) * Fraction(b), fmt)


def add(a, b, fmt=FP32):
    return rne(Fraction(a) + Fraction(b), fmt)


def rsqrt(m: Fraction, fmt=FP32) -> Fraction:
    """Correctly rounded 1 / sqrt(m) for m > 0.

    floor(2^k / sqrt(m)) comes from an integer square root; with k far above
    the format's precision the floor is within 2^-k of the exact value, so
    rounding it gives the correctly rounded result unless the exact value
    lies within 2^-k of a tie (then this raises: no FP32 input gets that
    close for k = 160 + the binade)."""
    m = Fraction(m)
    assert m > 0
    e = _floor_log2(1 / m) // 2
    k = 160 - e
    # 2^k / sqrt(m) = sqrt(2^(2k) / m)
    num = (1 << (2 * k)) * m.denominator
    r = math.isqrt(num // m.numerator)
    lo = Fraction(r, 1 << k)
    hi = Fraction(r + 1, 1 << k)
    a, b = rne(lo, fmt), rne(hi, fmt)
    if a != b:
        raise ArithmeticError("reciprocal square root too close to a tie")
    return a


def sqrt(m: Fraction, fmt=FP32) -> Fraction:
    """Correctly rounded sqrt(m) (same method as rsqrt)."""
    m = Fraction(m)
    assert m > 0
    e = _floor_log2(m) // 2
    k = 160 - e
    num = (1 << (2 * k)) * m.numerator
    r = math.isqrt(num // m.denominator)
    lo = Fraction(r, 1 << k)
    hi = Fraction(r + 1, 1 << k)
    a, b = rne(lo, fmt), rne(hi, fmt)
    if a != b:
        raise ArithmeticError("square root too close to a tie")
    return a


def div(a, b, fmt=FP32):
    return rne(Fraction(a) / Fraction(b), fmt)
