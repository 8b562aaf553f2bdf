"""Exact-rational model of the reduction, built from IEEE 754 definitions.

Used only to pin the oracle: it never touches the oracle's code, C floating
point or numpy rounding.  Values are ``fractions.Fraction``; rounding to a
binary format is done with integer arithmetic from the definition of
roundTiesToEven (IEEE 754-2019, 4.3.1): the representable value nearest to
the exact result, the one with an even last significand digit on a tie, and
overflow to infinity when the rounded magnitude reaches 2**(emax+1).
"""
from __future__ import annotations

from dataclasses import dataclass
from fractions import Fraction

INF = "inf"


@dataclass(frozen=True)
class Fmt:
    p: int      # significand precision in bits (with the implicit bit)
    emin: int
    emax: int
    ebits: int

    @property
    def bias(self) -> int:
        return self.emax


F32 = Fmt(p=24, emin=-126, emax=127, ebits=8)
BF16 = Fmt(p=8, emin=-126, emax=127, ebits=8)


def decode(bits: int, fmt: Fmt):
    """Bit pattern -> (sign, value) with value a Fraction, INF, or None (NaN)."""
    mbits = fmt.p - 1
    sign = (bits >> (fmt.ebits + mbits)) & 1
    e = (bits >> mbits) & ((1 << fmt.ebits) - 1)
    m = bits & ((1 << mbits) - 1)
    if e == (1 << fmt.ebits) - 1:
        return (sign, INF) if m == 0 else (sign, None)
    if e == 0:
        mag = Fraction(m) * Fraction(2) ** (fmt.emin - mbits)
    else:
        mag = Fraction((1 << mbits) | m) * Fraction(2) ** (e - fmt.bias - mbits)
    return sign, mag


def _floor_log2(q: Fraction) -> int:
    """floor(log2(q)) for q > 0."""
    e = q.numerator.bit_length() - q.denominator.bit_length()
    if Fraction(2) ** e > q:
        e -= 1
    if Fraction(2) ** (e + 1) <= q:
        e += 1
    return e


def round_rne(sign: int, mag, fmt: Fmt) -> int:
    """Round sign * mag (mag >= 0 Fraction, or INF) to fmt; return the bit pattern."""
    mbits = fmt.p - 1
    if mag == INF:
        return (sign << (fmt.ebits + mbits)) | (((1 << fmt.ebits) - 1) << mbits)
    if mag == 0:
        return sign << (fmt.ebits + mbits)
    e = max(_floor_log2(mag), fmt.emin)
    quantum = Fraction(2) ** (e - mbits)
    scaled = mag / quantum
    q = scaled.numerator // scaled.denominator
    rem = scaled - q
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and q % 2 == 1):
        q += 1
    value = q * quantum
    if value >= Fraction(2) ** (fmt.emax + 1):
        return round_rne(sign, INF, fmt)
    if value < Fraction(2) ** fmt.emin:          # subnormal (or zero after rounding)
        field_e, field_m = 0, int(value / Fraction(2) ** (fmt.emin - mbits))
    else:
        ee = _floor_log2(value)
        field_e = ee + fmt.bias
        field_m = int(value / Fraction(2) ** (ee - mbits)) - (1 << mbits)
    return (sign << (fmt.ebits + mbits)) | (field_e << mbits) | field_m


def add_rne(a, b, fmt: Fmt):
    """IEEE addition of two decoded operands (sign, mag) in fmt; returns (sign, mag).

    Exact zero sums take +0 unless both operands are -0 (IEEE 754-2019, 6.3).
    NaN is returned as (0, None).
    """
    (sa, ma), (sb, mb) = a, b
    if ma is None or mb is None:
        return (0, None)
    if ma == INF or mb == INF:
        if ma == INF and mb == INF and sa != sb:
            return (0, None)
        return (sa, INF) if ma == INF else (sb, INF)
    exact = (-ma if sa else ma) + (-mb if sb else mb)
    if exact == 0:
        return (1 if (sa and sb) else 0, Fraction(0))
    sign = 1 if exact < 0 else 0
    bits = round_rne(sign, abs(exact), fmt)
    return decode(bits, fmt)


def reduce_element(values_bf16, nan_bits: int = 0x7FC0) -> int:
    """bf16 result of sum in rank order, binary32 accumulation, RNE to bf16."""
    acc = decode(values_bf16[0], BF16)
    for v in values_bf16[1:]:
        acc = add_rne(acc, decode(v, BF16), F32)
    sign, mag = acc
    if mag is None:
        return nan_bits
    return round_rne(sign, mag, BF16)
