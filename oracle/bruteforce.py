"""Exact rational brute force for tiny inputs (pins the fp64 oracle).

TEST INFRASTRUCTURE, like the rest of this package: only the test-suite may
use it.

bf16 and fp32 inputs are dyadic rationals, so every product and sum in the
DoRA row norm [P2 "The Problem": ||W + sBA||_row] and in the compose
[P1 "DoRA优化技术解析" §2.1] is computed here exactly with
``fractions.Fraction``; the square root is taken to 50 significant digits
with ``decimal``. Nothing here uses floating-point arithmetic on results.
"""

from __future__ import annotations

from decimal import Decimal, getcontext
from fractions import Fraction

__all__ = ["exact_row_sq_norms", "exact_sqrt", "exact_compose", "round_fraction_bf16", "round_fraction_f16",
           "round_fraction_f32", "exact_compose_f32_stable", "exact_compose_f32_naive"]


def _fr(v) -> Fraction:
    return Fraction(float(v))


def exact_row_sq_norms(W, A, B, s):
    """sum_k (W[j,k] + s * sum_l B[j,l] A[l,k])^2 for every row j, exactly."""
    d_out = len(W)
    d_in = len(W[0]) if d_out else 0
    r = len(A)
    sf = _fr(s)
    Af = [[_fr(A[l][k]) for k in range(d_in)] for l in range(r)]
    out = []
    for j in range(d_out):
        Bj = [_fr(B[j][l]) for l in range(r)]
        acc = Fraction(0)
        for k in range(d_in):
            ba = sum((Bj[l] * Af[l][k] for l in range(r)), Fraction(0))
            v = _fr(W[j][k]) + sf * ba
            acc += v * v
        out.append(acc)
    return out


def exact_sqrt(q: Fraction, digits: int = 50) -> Decimal:
    """Square root of a non-negative rational to ``digits`` significant digits."""
    getcontext().prec = digits + 10
    return (Decimal(q.numerator) / Decimal(q.denominator)).sqrt()


def exact_compose(base, lora, g, s):
    """(g-1)*base + g*(s*lora) for one element, exactly."""
    gf = _fr(g)
    return (gf - 1) * _fr(base) + gf * (_fr(s) * _fr(lora))


def round_fraction_bf16(q: Fraction) -> Fraction:
    """Round an exact rational to bfloat16 (8 significant bits), ties to even.

    Independent of the oracle's float-based rounding: the binade is found by
    exact comparison with powers of two and the tie is decided on integers.
    Handles the normal range only (the tests never leave it).
    """
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = 0
    while a >= 2 ** (e + 1):
        e += 1
    while a < Fraction(2) ** e:
        e -= 1
    # a in [2^e, 2^(e+1)); spacing 2^(e-7)
    spacing = Fraction(2) ** (e - 7)
    n = a / spacing                       # in [128, 256)
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * spacing


def round_fraction_f16(q: Fraction):
    """Round an exact rational to IEEE binary16, ties to even, on integers.

    11 significant bits in the normal range (exponents -14 .. 15), a fixed
    spacing of 2^-24 below 2^-14 (subnormals), and +-inf at or beyond the
    midpoint 65520 between the largest finite value 65504 and 2^16.
    Returns a Fraction, or +-float('inf').
    """
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = 0
    while a >= 2 ** (e + 1):
        e += 1
    while a < Fraction(2) ** e:
        e -= 1
    spacing = Fraction(2) ** (max(e, -14) - 10)
    n = a / spacing
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    v = fl * spacing
    if v > 65504:
        return sign * float("inf")
    return sign * v


def round_fraction_f32(q: Fraction):
    """Round an exact rational to IEEE binary32, ties to even, on integers.

    24 significant bits in the normal range (exponents -126 .. 127), a fixed
    spacing of 2^-149 below 2^-126 (subnormals), and +-inf once the rounded
    magnitude reaches 2^128 (the midpoint between the largest finite value
    2^128 - 2^104 and 2^128 rounds to the even neighbour, 2^128, so to inf).
    Returns a Fraction, or +-float('inf'). Independent of numpy's casts.
    """
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = 0
    while a >= Fraction(2) ** (e + 1):
        e += 1
    while a < Fraction(2) ** e:
        e -= 1
    spacing = Fraction(2) ** (max(e, -126) - 23)
    n = a / spacing
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    v = fl * spacing
    if v >= Fraction(2) ** 128:
        return sign * float("inf")
    return sign * v


def _r32(q: Fraction) -> Fraction:
    v = round_fraction_f32(q)
    if not isinstance(v, Fraction):
        raise OverflowError("binary32 overflow in an exact per-operation evaluation")
    return v


def exact_compose_f32_stable(base, lora, g, s) -> Fraction:
    """The stable compose (g - 1) * base + g * (s * lora) evaluated as binary32
    arithmetic does it, one element: every input rounded to binary32, then
    s * lora, g - 1, (g - 1) * base, g * (s * lora) and the final sum, each
    computed exactly and rounded once to binary32 (round to nearest even)."""
    b, l, gg, sf = (_r32(_fr(v)) for v in (base, lora, g, s))
    sl = _r32(sf * l)
    p1 = _r32(_r32(gg - 1) * b)
    p2 = _r32(gg * sl)
    return _r32(p1 + p2)


def exact_compose_f32_naive(base, lora, g, s) -> Fraction:
    """The naive compose g * (s * lora + base) - base in binary32 arithmetic,
    one element, with the same per-operation rounding as above."""
    b, l, gg, sf = (_r32(_fr(v)) for v in (base, lora, g, s))
    t = _r32(_r32(sf * l) + b)
    return _r32(_r32(gg * t) - b)
