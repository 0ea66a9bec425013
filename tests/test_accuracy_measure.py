"""The correct-bits measure used by the benchmark and the accuracy sweep is
checked against the oracle's exact computation and against hand-made cases."""
import math

import numpy as np
import pytest

from fp64_gemm_emulation_ozii_amd import accuracy as acc
from oracle import ozaki2 as oz


def test_exact_sum_matches_oracle():
    rng = np.random.default_rng(5)
    for n in [1, 7, 300]:
        a = (rng.random(n) - 0.5) * np.exp(4 * rng.standard_normal(n))
        b = (rng.random(n) - 0.5) * np.exp(4 * rng.standard_normal(n))
        a[::5] = 0.0
        N1, p1 = acc._exact_sum_products(a, b)
        N2, p2 = oz.exact_dot(a, b)
        # same value, possibly different normalisation
        e = min(p1, p2)
        assert (N1 << (p1 - e)) == (N2 << (p2 - e))


def test_subnormal_and_huge_terms():
    a = np.array([5e-324, 1e300, -1e300, 3.0])
    b = np.array([2.0, 1e8, 1e8, 0.5])
    N, p = acc._exact_sum_products(a, b)
    from fractions import Fraction
    assert Fraction(N) * Fraction(2) ** p == Fraction(5e-324) * 2 + Fraction(3.0) * Fraction(0.5)


def test_correct_bits_matches_oracle():
    rng = np.random.default_rng(9)
    A = (rng.random((6, 50)) - 0.5) * np.exp(rng.standard_normal((6, 50)))
    B = (rng.random((50, 5)) - 0.5) * np.exp(rng.standard_normal((50, 5)))
    C = A @ B
    C[2, 3] += 1e-9
    rows, cols = np.arange(6).repeat(5), np.tile(np.arange(5), 6)
    vals = C[rows, cols]
    assert acc.correct_bits(vals, A, B, rows, cols) == pytest.approx(oz.correct_bits(C, A, B, rows, cols), abs=1e-12)


def test_correct_bits_known_values():
    A = np.array([[1.0, 1.0]])
    B = np.array([[1.0], [-1.0]])
    # exact product 0, |A||B| = 2: an error of 2^-40 gives 41 bits
    assert acc.correct_bits([2.0 ** -40], A, B, [0], [0]) == pytest.approx(41.0)
    assert acc.correct_bits([0.0], A, B, [0], [0]) == 64.0
    assert acc.correct_bits([math.nan], A, B, [0], [0]) < 0


@pytest.mark.parametrize("phi", [0.5, 2.0, 16.0])
def test_compensated_measure_matches_the_exact_one(phi):
    """correct_bits_many (compensated dot products, thousands of entries) gives
    the exact measure's figure to well under 0.01 bit, for exact, slightly
    perturbed and coarsely wrong values."""
    rng = np.random.default_rng(int(phi * 10))
    A = (rng.random((9, 700)) - 0.5) * np.exp(phi * rng.standard_normal((9, 700)))
    B = (rng.random((700, 8)) - 0.5) * np.exp(phi * rng.standard_normal((700, 8)))
    A[3, ::4] = 0.0
    rows, cols = np.arange(9).repeat(8), np.tile(np.arange(8), 9)
    C = A @ B
    for scale in (0.0, 2.0**-50, 2.0**-30):
        vals = C[rows, cols] + scale * (np.abs(A) @ np.abs(B))[rows, cols] * rng.standard_normal(len(rows))
        exact = acc.correct_bits(vals, A, B, rows, cols)
        fast = acc.correct_bits_many(vals, A, B, rows, cols)
        assert fast == pytest.approx(exact, abs=0.01), (scale, exact, fast)
    bad = C[rows, cols].copy()
    bad[5] = np.inf
    assert acc.correct_bits_many(bad, A, B, rows, cols) == 0.0
