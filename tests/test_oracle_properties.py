"""Property tests of the oracle over random inputs (hypothesis), each against
something other than the oracle itself: exact rational arithmetic, integer
arithmetic or an independent library routine."""
import math
from fractions import Fraction

import numpy as np
import pytest

hyp = pytest.importorskip("hypothesis")
from hypothesis import given, settings, strategies as st
from hypothesis.extra import numpy as hnp


@pytest.fixture(scope="module")
def orc():
    import oracle
    oracle.lib()
    return oracle


finite32 = st.floats(width=32, allow_nan=False, allow_infinity=False)


@settings(max_examples=200, deadline=None)
@given(st.lists(st.lists(finite32, min_size=3, max_size=3), min_size=1, max_size=12))
def test_reduce_is_the_exactly_rounded_sum(orc, rows):
    """oracle.reduce: each element is the exact sum of the fp32 sources
    rounded once to double, as the rational sum (Fraction) and math.fsum
    give it."""
    srcs = [np.array(r, dtype=np.float32) for r in rows]
    got = orc.reduce(srcs)
    for j in range(3):
        exact = sum(Fraction(float(s[j])) for s in srcs)
        assert float(got[j]) == float(exact), j                   # Fraction -> float rounds once
        assert float(got[j]) == math.fsum(float(s[j]) for s in srcs)


@settings(max_examples=100, deadline=None)
@given(st.integers(1, 9), st.integers(1, 9), st.integers(1, 40), st.integers(0, 2 ** 31 - 1))
def test_gemm_integer_inputs_equal_int64(orc, m, n, k, seed):
    """Integer-valued bf16 operands: the fp64 oracle equals int64 matmul."""
    g = np.random.Generator(np.random.PCG64(seed))
    xi = g.integers(-3, 4, size=(m, k))
    wi = g.integers(-3, 4, size=(n, k))
    to_bits = lambda a: (np.asarray(a, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
    got = orc.gemm(to_bits(xi), to_bits(wi))
    assert np.array_equal(got, (xi @ wi.T).astype(np.float64))


@settings(max_examples=60, deadline=None)
@given(st.integers(1, 4), st.integers(1, 4), st.integers(1, 6), st.integers(0, 2 ** 31 - 1))
def test_gemm_fractional_inputs_equal_fraction_sum(orc, m, n, k, seed):
    """bf16 operands with random signs and mantissas and exponents within
    2^-4 .. 2^4, on tiny shapes: every product (16 significant bits) and
    every partial sum then fits a double exactly, so the oracle's fp64
    result equals the exact rational dot product."""
    g = np.random.Generator(np.random.PCG64(seed))

    def operand(shape):
        sign = g.integers(0, 2, size=shape) << 15
        expo = g.integers(127 - 4, 127 + 5, size=shape) << 7
        mant = g.integers(0, 128, size=shape)
        return (sign | expo | mant).astype(np.uint16)

    xb, wb = operand((m, k)), operand((n, k))
    dec = lambda b: float(np.array([int(b) << 16], dtype=np.uint32).view(np.float32)[0])
    got = orc.gemm(xb, wb)
    for i in range(m):
        for j in range(n):
            exact = sum(Fraction(dec(xb[i, t])) * Fraction(dec(wb[j, t])) for t in range(k))
            assert got[i, j] == float(exact), (i, j)


@settings(max_examples=300, deadline=None)
@given(st.floats(allow_nan=False, allow_infinity=False, min_value=-3e38, max_value=3e38))
def test_f64_to_bf16_is_nearest_even(orc, v):
    """Round to nearest, ties to even, checked with exact rationals against
    the two bf16 neighbours of v."""
    bits = int(orc.f64_to_bf16(np.array([v]))[0])
    dec = lambda b: float(np.array([b << 16], dtype=np.uint32).view(np.float32)[0])
    r = dec(bits)
    if math.isinf(r):
        return                                      # beyond the largest bf16: overflow to infinity
    fv = Fraction(v)
    # the neighbours one bf16 ulp away on each side
    up = dec((bits + 1) & 0xFFFF) if (bits & 0x7FFF) != 0x7F7F else math.inf
    dn = dec((bits - 1) & 0xFFFF) if (bits & 0x7FFF) != 0 else -dec(bits) if r == 0 else dec(bits - 1)
    err = abs(Fraction(r) - fv)
    for nb in (up, dn):
        if math.isinf(nb):
            continue
        d = abs(Fraction(nb) - fv)
        assert err < d or (err == d and (bits & 1) == 0), (v, r, nb)
