"""Exact rational brute force for tiny shapes (TEST INFRASTRUCTURE).

Decodes bf16 bit patterns from their sign / exponent / fraction fields into
``fractions.Fraction`` values (a decode path independent of the C oracle's)
and evaluates the same definitions with exact rational arithmetic: the
product Y = X * W and element-wise sums.  Used only to pin the fp64 oracle on
shapes with every dimension of about 16 or less.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np


def bf16_fraction(bits: int) -> Fraction:
    """Exact value of a finite bf16 bit pattern."""
    bits = int(bits) & 0xFFFF
    sign = -1 if bits >> 15 else 1
    exp = (bits >> 7) & 0xFF
    frac = bits & 0x7F
    if exp == 0xFF:
        raise ValueError("not finite")
    if exp == 0:                      # subnormal: frac * 2^-133
        mag = Fraction(frac, 2 ** 133)
    else:                             # (128 + frac) * 2^(exp - 127 - 7)
        e = exp - 134
        mag = Fraction(128 + frac) * (Fraction(2) ** e)
    return sign * mag


def f32_fraction(x: float) -> Fraction:
    return Fraction(float(np.float32(x)))


def gemm(x_bits: np.ndarray, w_bits: np.ndarray):
    """Exact Y[i][j] = sum_t X[i][t] * W[j][t] (W stored [n][k])."""
    m, k = x_bits.shape
    n = w_bits.shape[0]
    X = [[bf16_fraction(x_bits[i, t]) for t in range(k)] for i in range(m)]
    W = [[bf16_fraction(w_bits[j, t]) for t in range(k)] for j in range(n)]
    return [[sum((X[i][t] * W[j][t] for t in range(k)), Fraction(0))
             for j in range(n)] for i in range(m)]


def sum_exact(values) -> Fraction:
    return sum((Fraction(float(v)) for v in values), Fraction(0))


def to_float(F) -> np.ndarray:
    """Round a nested list of Fractions to float64 (Fraction -> float is
    correctly rounded)."""
    return np.array([[float(v) for v in row] for row in F], dtype=np.float64)
