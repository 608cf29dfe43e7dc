"""Independent arithmetic used to pin the oracle (test code only).

Nothing here is shared with the oracle or with the GPU library.  Exact values
come from ``fractions.Fraction``, square roots from ``decimal`` at 60 digits,
binary32 sums from numpy float32 scalars, and bit-pattern decoding from numpy
views (a different implementation from the oracle's decoder).
"""
from __future__ import annotations

import math
from decimal import Decimal, localcontext
from fractions import Fraction

import numpy as np

# (significand bits incl. the implicit one, min normal exponent, max exponent)
FORMATS = {"f32": (24, -126, 127), "f16": (11, -14, 15), "bf16": (8, -126, 127)}
INF = float("inf")


def decode_np(a: np.ndarray, dtype: str) -> np.ndarray:
    """Storage -> float64 through numpy views (independent of the oracle)."""
    if dtype == "f32":
        return a.astype(np.float64)
    if dtype == "f16":
        return a.view(np.float16).astype(np.float64)
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def floor_log2(a: Fraction) -> int:
    """Largest e with 2^e <= a (a > 0), by integer arithmetic."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    if Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def exact_round(q: Fraction, dtype: str):
    """Round an exact rational to dtype: nearest, ties to even, overflow to inf.

    Returns (value, tie_distance) where value is a Fraction (or +-inf) and
    tie_distance = |fractional part - 1/2| in units of the quantum (0 means an
    exact tie; a tiny value means the input sits next to a rounding boundary).
    """
    p, emin, emax = FORMATS[dtype]
    if q == 0:
        return Fraction(0), Fraction(1, 2)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = max(floor_log2(a), emin)
    quantum = Fraction(2) ** (e - (p - 1))
    n = a / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * quantum
    maxfin = (2 ** p - 1) * Fraction(2) ** (emax - (p - 1))
    if r > maxfin:
        return sign * INF, abs(rem - Fraction(1, 2))
    return sign * r, abs(rem - Fraction(1, 2))


def storage_of(value, dtype: str):
    """Bit pattern / float32 of a value exactly representable in dtype."""
    f = float(value)
    if dtype == "f32":
        return np.float32(f)
    if dtype == "f16":
        return np.array([f], dtype=np.float16).view(np.uint16)[0]
    b = np.array([f], dtype=np.float32).view(np.uint32)[0]
    assert b & 0xFFFF == 0, "value not representable in bf16"
    return np.uint16(b >> 16)


def dec(q: Fraction) -> Decimal:
    return Decimal(q.numerator) / Decimal(q.denominator)


def fused_residual_f32(vals):
    """Binary32 sum of the values in the given order, seeded with the first."""
    acc = np.float32(vals[0])
    for v in vals[1:]:
        acc = np.float32(acc + np.float32(v))
    return acc


def round_signed(q: Fraction, sign_src: float, dtype: str):
    """exact_round, returned as a Python float with IEEE signed zeros: a result
    that is zero takes the sign of ``sign_src``."""
    r, tie = exact_round(q, dtype)
    if r == 0:
        return math.copysign(0.0, sign_src), tie
    return float(r), tie


def bits(value: float, dtype: str) -> int:
    """Bit pattern (as int) of a float exactly representable in dtype."""
    s = storage_of(value, dtype)
    if dtype == "f32":
        return int(np.array([s], dtype=np.float32).view(np.uint32)[0])
    return int(s)


def storage_bits(a: np.ndarray, dtype: str) -> np.ndarray:
    return a.view(np.uint32) if dtype == "f32" else a


def brute_force_row(v_row, gamma_row, eps: float, dtype: str):
    """Exact RMSNorm of one row.  v_row, gamma_row: float values (signed zeros
    allowed); eps: the float32 argument.  The sum of squares and the mean are
    exact rationals, the square root and reciprocal 60-digit decimals.
    Returns [(rounded float, tie_distance)] per element; a zero product takes
    the IEEE sign of v * gamma."""
    H = len(v_row)
    vs = [Fraction(float(v)) for v in v_row]
    ms = sum(v * v for v in vs) / H
    denom = ms + Fraction(float(np.float32(eps)))
    out = []
    with localcontext() as ctx:
        ctx.prec = 60
        inv = Decimal(1) / dec(denom).sqrt()
        for v, vf, g in zip(vs, v_row, gamma_row):
            y = dec(v) * inv * dec(Fraction(float(g)))
            sign = math.copysign(1.0, float(vf)) * math.copysign(1.0, float(g))
            if y != 0:
                sign = 1.0 if y > 0 else -1.0
            out.append(round_signed(Fraction(y), sign, dtype))
    return out


def ulp_distance(a_bits: np.ndarray, b_bits: np.ndarray, dtype: str) -> np.ndarray:
    """Distance in units in the last place between two arrays of storage
    (monotone integer mapping of the bit patterns; +0 and -0 coincide)."""
    if dtype == "f32":
        ia = a_bits.view(np.int32).astype(np.int64)
        ib = b_bits.view(np.int32).astype(np.int64)
        ia = np.where(ia < 0, -(ia & 0x7FFFFFFF), ia)
        ib = np.where(ib < 0, -(ib & 0x7FFFFFFF), ib)
    else:
        ia = a_bits.view(np.int16).astype(np.int64)
        ib = b_bits.view(np.int16).astype(np.int64)
        ia = np.where(ia < 0, -(ia & 0x7FFF), ia)
        ib = np.where(ib < 0, -(ib & 0x7FFF), ib)
    return np.abs(ia - ib)


def isclose_rel(a: float, b: float, rel: float) -> bool:
    if a == b:
        return True
    return abs(a - b) <= rel * max(abs(a), abs(b))


def sqrt_dec(q: Fraction) -> Decimal:
    with localcontext() as ctx:
        ctx.prec = 60
        return dec(q).sqrt()


__all__ = [n for n in dir() if not n.startswith("_")] + ["math"]
