"""Exact rational helpers for pinning the oracle (tests only).

Everything here is computed with Python integers and fractions from the
IEEE 754 definitions, independently of numpy's floating-point arithmetic,
so that the oracle can be checked against something other than itself.
"""
from __future__ import annotations

from fractions import Fraction
from math import floor


def f16_value(bits: int) -> Fraction | None:
    """Exact value of an IEEE binary16 pattern; None for inf/NaN."""
    s = (bits >> 15) & 1
    e = (bits >> 10) & 0x1F
    m = bits & 0x3FF
    if e == 0x1F:
        return None
    if e == 0:
        v = Fraction(m, 1 << 10) * Fraction(1, 1 << 14)
    else:
        v = (1 + Fraction(m, 1 << 10)) * (Fraction(2) ** (e - 15))
    return -v if s else v


def f32_value(bits: int) -> Fraction | None:
    """Exact value of an IEEE binary32 pattern; None for inf/NaN."""
    s = (bits >> 31) & 1
    e = (bits >> 23) & 0xFF
    m = bits & 0x7FFFFF
    if e == 0xFF:
        return None
    if e == 0:
        v = Fraction(m, 1 << 23) * (Fraction(2) ** -126)
    else:
        v = (1 + Fraction(m, 1 << 23)) * (Fraction(2) ** (e - 127))
    return -v if s else v


def bf16_value(bits: int) -> Fraction | None:
    return f32_value((bits & 0xFFFF) << 16)


def round_to_binary32(v: Fraction) -> Fraction:
    """Round an exact rational to the nearest binary32 value, ties to even."""
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    quantum = Fraction(2) ** (e - 23)
    n = a / quantum
    fl = floor(n)
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * quantum
    if r >= Fraction(2) ** 128:
        raise OverflowError
    return sign * r


def round_to_bf16(v: Fraction) -> Fraction:
    """Round an exact rational (a binary32 value) to bf16, ties to even."""
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    quantum = Fraction(2) ** (e - 7)
    n = a / quantum
    fl = floor(n)
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * quantum


def decode_nibble_rule(u: int, enc: str) -> int:
    """The decode rules as the pages state them, one value at a time."""
    if enc == "twos":
        return u if u < 8 else u - 16
    return u - 8


def unpack_byte_rows(packed_rows, K: int, enc: str):
    """Literal per-byte unpack: byte b -> columns 2b (bits 0-3), 2b+1 (bits 4-7)."""
    rows = []
    for row in packed_rows:
        codes = []
        for b in row:
            b = int(b)
            codes.append(decode_nibble_rule(b & 0xF, enc))
            codes.append(decode_nibble_rule((b >> 4) & 0xF, enc))
        rows.append(codes[:K])
    return rows


def exact_matmul_dequant(x_vals, w_vals):
    """Textbook y[m][n] = sum_k x[m][k] * W[n][k] over exact fractions."""
    return [[sum((xv * wv for xv, wv in zip(xr, wr)), Fraction(0)) for wr in w_vals] for xr in x_vals]
