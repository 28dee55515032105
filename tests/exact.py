"""Exact rational helpers for pinning the oracle (independent of it).

Correct rounding of a rational number to fp32 / bf16 is written here from
the IEEE-754 definition (nearest representable value, ties to the even
significand, gradual underflow, overflow to infinity), so tests can compare
the oracle's fp32 steps against the mathematically exact result.
"""
from __future__ import annotations

import struct
from fractions import Fraction

import numpy as np

F32_MAX = Fraction(2) ** 127 * (2 - Fraction(1, 2 ** 23))


def _round_half_even(q: Fraction) -> int:
    n = q.numerator // q.denominator
    r = q - n
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return n


def to_f32(q: Fraction) -> float:
    """Nearest fp32 to the rational q (ties to even), as a Python float."""
    if q == 0:
        return 0.0
    sign = -1.0 if q < 0 else 1.0
    a = abs(q)
    # exponent e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    if e >= -126:
        step = Fraction(2) ** (e - 23)
    else:
        step = Fraction(2) ** -149
    m = _round_half_even(a / step)
    val = m * step
    if val > F32_MAX:
        return sign * float("inf")
    return sign * float(val)


def f32(x: float) -> np.float32:
    return np.float32(x)


def f32_bits(x) -> int:
    return struct.unpack("<I", struct.pack("<f", float(np.float32(x))))[0]


def bits_f32(u: int) -> float:
    return struct.unpack("<f", struct.pack("<I", u & 0xFFFFFFFF))[0]


def bf16_values_nonneg_finite() -> np.ndarray:
    """All finite, non-negative bf16 values as fp32 (includes +0 and subnormals)."""
    h = np.arange(0, 0x7F80, dtype=np.uint32)
    return (h << 16).view(np.float32)


def grid_values(grid: int):
    """Element grids written as sets: E2M1 (OCP FP4 table) and uniform INT4."""
    if grid == 0:
        return [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
                Fraction(4), Fraction(6)]
    return [Fraction(k) for k in range(8)]


def bracket(grid: int, v: Fraction):
    """(k_lo, k_hi) of the clamped value by brute force over the grid."""
    G = grid_values(grid)
    vc = min(v, G[-1])
    klo = max(k for k in range(8) if G[k] <= vc)
    khi = min(k for k in range(8) if G[k] >= vc)
    return klo, khi, vc
