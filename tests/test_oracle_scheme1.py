"""Pins of the Scheme I oracle (oracle/ozaki1.py) against what the Ozaki I and
Ozaki II notes fix and against the mathematics, independent of the oracle's
own formulas."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import ozaki1 as o1

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "ozaki_page_facts.json")))


# ---------------------------------------------------------------- parameters

@pytest.mark.parametrize("case", GOLDEN["rn_split_slice_width"]["cases"])
def test_beta_and_r_match_page_values(case):
    beta = o1.slice_width(case["n"])
    assert beta == case["beta"]
    assert o1.group_size(case["n"], beta) == case["r"]


@pytest.mark.parametrize("q", [1, 2, 3, 100, 1000, 4095, 4097, 12345, 2**17 - 1, 2**17 + 1, 10**6, 2**21 + 7])
def test_beta_equals_real_formula_away_from_boundaries(q):
    real = math.floor((31 - math.log2(q)) / 2)
    assert o1.slice_width(q) == min(7, real)
    beta = o1.slice_width(q)
    assert o1.group_size(q, beta) == max(1, 2 ** (31 - 2 * beta - math.ceil(math.log2(q))))


def test_beta_keeps_int32_exact():
    for q in [1, 64, 4096, 65536, 2**20, 2**23]:
        b = o1.slice_width(q)
        # q products of magnitude at most 2^(b-1) * 2^(b-1), summed r at a time
        assert q * 4 ** (b - 1) * o1.group_size(q, b) < 2**31


@pytest.mark.parametrize("k,count", sorted((int(a), b) for a, b in GOLDEN["scheme1_gemm_count"]["slices_to_gemms"].items()))
def test_triangle_count_matches_page_table(k, count):
    pairs = o1.triangle(k)
    assert len(pairs) == count
    assert len(set(pairs)) == count
    assert all(i + j <= k + 1 and i >= 1 and j >= 1 for i, j in pairs)
    # i-major, j-minor
    assert pairs == sorted(pairs)


@pytest.mark.parametrize("k", [1, 2, 4, 8, 10])
@pytest.mark.parametrize("r", [1, 2, 3, 32])
def test_groups_cover_triangle_once(k, r):
    gs = o1.groups(k, r)
    flat = [p for _, run in gs for p in run]
    assert sorted(flat) == sorted(o1.triangle(k))
    assert len(flat) == len(set(flat))
    for g, run in gs:
        assert 1 <= len(run) <= r
        assert all(s + t == g for s, t in run)
    assert [g for g, _ in gs] == sorted(g for g, _ in gs)


# ------------------------------------------------------------------- the split

def _rows(seed, rows=6, cols=40, phi=1.0):
    rng = np.random.default_rng(seed)
    X = (rng.random((rows, cols)) - 0.5) * np.exp(phi * rng.standard_normal((rows, cols)))
    X[1, :] *= 2.0**-30
    X[2, :] *= 2.0**40
    X[3, 5] = 0.0
    X[4, :] = 0.0
    return X


def test_magic_constant_literal_equals_grid_rounding():
    """(a + sigma) - sigma with sigma = 0.75 2^53 mu, evaluated as the notes
    write it, equals the oracle's rounding to the mu grid (RN split step 5)."""
    X = _rows(1)
    beta = 7
    E, zero, _ = o1._ceil_log2_rows(X)
    g = np.where(zero, 0, E + 1 - beta)
    mu = np.ldexp(1.0, g)
    sigma = 0.75 * 2.0**53 * mu
    literal = (X + sigma[:, None]) - sigma[:, None]
    ours = np.ldexp(o1._round_to_grid(X, g), g[:, None])
    assert np.array_equal(literal, ours)


def test_magic_constant_needs_factor_one_and_a_half():
    """The notes: with sigma = 2^52 mu, negative a lands on a half-grid;
    1.5 2^52 mu rounds both signs to the grid."""
    a = np.array([-3.3, -0.75, -2.5, 2.5, 3.5, -3.5, 0.49])
    good = (a + 1.5 * 2.0**52) - 1.5 * 2.0**52
    bad = (a + 2.0**52) - 2.0**52
    assert np.array_equal(good, np.rint(a))
    assert not np.array_equal(bad, np.rint(a))


@pytest.mark.parametrize("variant", ["rn", "hybrid"])
@pytest.mark.parametrize("k", [1, 3, 6])
def test_split_is_exact_decomposition(variant, k):
    X = _rows(2 + k)
    beta = 7
    if variant == "rn":
        sl, ge, bad = o1.split_rn(X, k, beta)
        grids = ge
    else:
        sl, g0, bad = o1.split_hybrid(X, k, beta)
        grids = np.stack([g0 - beta * p for p in range(k)])
    assert not bad.any()
    assert np.all(np.abs(sl.astype(int)) <= 2 ** (beta - 1))
    for i in range(X.shape[0]):
        E = o1._ceil_log2_rows(X[i:i + 1])[0][0]
        for j in range(X.shape[1]):
            rec = sum(Fraction(int(sl[p, i, j])) * Fraction(2) ** int(grids[p, i]) for p in range(k))
            err = Fraction(float(X[i, j])) - rec
            if X[i].any():
                # the residual after k slices is at most half the last grid
                assert abs(err) <= Fraction(2) ** int(grids[k - 1, i]) / 2
                assert abs(err) <= Fraction(2) ** int(E - beta * k)
            else:
                assert err == 0 and rec == 0


def test_rn_split_grid_follows_residual():
    """RN split: each grid is 2^(ceil(log2 max|R|) + 1 - beta) of the residual
    left by the previous slices (RN split algorithm step 3)."""
    X = _rows(7)
    beta, k = 7, 4
    sl, ge, _ = o1.split_rn(X, k, beta)
    R = [[Fraction(float(v)) for v in row] for row in X]
    for p in range(k):
        for i in range(X.shape[0]):
            mx = max(abs(v) for v in R[i])
            if mx == 0:
                continue
            E = 0  # exact ceil(log2 mx) of a rational
            while Fraction(2) ** E < mx:
                E += 1
            while Fraction(2) ** (E - 1) >= mx:
                E -= 1
            assert ge[p, i] == E + 1 - beta
            for j in range(X.shape[1]):
                R[i][j] -= Fraction(int(sl[p, i, j])) * Fraction(2) ** int(ge[p, i])


# --------------------------------------------------------------- whole product

@pytest.mark.parametrize("variant", ["rn", "hybrid"])
@pytest.mark.parametrize("k", [1, 2, 5])
def test_small_integer_inputs_give_textbook_product(variant, k):
    rng = np.random.default_rng(11 + k)
    A = rng.integers(-63, 64, size=(9, 33)).astype(np.float64)
    B = rng.integers(-63, 64, size=(33, 7)).astype(np.float64)
    A[:, 0] = 63.0  # every row reaches 2^6 - 1 -> first slice holds it exactly
    B[0, :] = -63.0
    C = o1.dgemm(A, B, k, variant)
    assert np.array_equal(C, (A.astype(np.int64) @ B.astype(np.int64)).astype(np.float64))


@pytest.mark.parametrize("variant", ["rn", "hybrid"])
def test_identity_reproduces_b(variant):
    rng = np.random.default_rng(5)
    n = 24
    B = (0.5 + 0.5 * rng.random((n, 11))) * rng.choice([-1.0, 1.0], size=(n, 11))
    C = o1.dgemm(np.eye(n), B, 8, variant)
    assert np.array_equal(C, B)


def test_zero_and_nonfinite_rows():
    rng = np.random.default_rng(3)
    A = rng.standard_normal((5, 16))
    B = rng.standard_normal((16, 4))
    A[1, :] = 0.0
    A[2, 3] = np.inf
    B[5, 2] = np.nan
    for v in ["rn", "hybrid"]:
        C = o1.dgemm(A, B, 5, v)
        assert np.all(C[1, [0, 1, 3]] == 0.0)
        assert np.all(np.isnan(C[2, :]))
        assert np.all(np.isnan(C[:, 2]))
        assert np.all(np.isfinite(C[[0, 3, 4]][:, [0, 1, 3]]))


def _exact_err_bits(C, A, B):
    worst = Fraction(0)
    for i in range(A.shape[0]):
        for j in range(B.shape[1]):
            ex = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(A[i], B[:, j]))
            den = sum(abs(Fraction(float(a)) * Fraction(float(b))) for a, b in zip(A[i], B[:, j]))
            if den:
                worst = max(worst, abs(Fraction(float(C[i, j])) - ex) / den)
    return 64.0 if worst == 0 else -math.log2(worst)


@pytest.mark.parametrize("variant", ["rn", "hybrid"])
def test_accuracy_grows_with_slices(variant):
    rng = np.random.default_rng(21)
    A = (rng.random((6, 48)) - 0.5) * np.exp(0.5 * rng.standard_normal((6, 48)))
    B = (rng.random((48, 5)) - 0.5) * np.exp(0.5 * rng.standard_normal((48, 5)))
    bits = [_exact_err_bits(o1.dgemm(A, B, k, variant), A, B) for k in range(2, 9)]
    # about beta = 7 bits per slice until FP64 rounding takes over
    for a, b in zip(bits[:4], bits[1:5]):
        assert b >= a + 4.0
    assert bits[-1] >= 50.0


def test_group_sums_equal_products_of_the_same_slices():
    rng = np.random.default_rng(8)
    A = rng.standard_normal((7, 20))
    B = rng.standard_normal((20, 6))
    C, st = o1.dgemm(A, B, 6, "hybrid", stages=True)
    for (g, run), P in zip(st["groups"], st["products"]):
        direct = sum(st["As"][s - 1].astype(np.int64) @ st["Bs"][t - 1].astype(np.int64) for s, t in run)
        assert np.array_equal(P, direct)


def test_rn_terms_accumulate_in_triangle_order():
    """Re-adding the stored products in the documented order reproduces C
    bit for bit; another order generally does not."""
    rng = np.random.default_rng(9)
    A = (rng.random((8, 30)) - 0.5) * np.exp(2 * rng.standard_normal((8, 30)))
    B = (rng.random((30, 8)) - 0.5) * np.exp(2 * rng.standard_normal((30, 8)))
    C, st = o1.dgemm(A, B, 5, "rn", stages=True)
    acc = np.zeros_like(C)
    for (i, j), P in zip(st["pairs"], st["products"]):
        acc = acc + np.ldexp(P.astype(float), st["gA"][i - 1][:, None] + st["gB"][j - 1][None, :])
    assert np.array_equal(acc, C)


# --------------------------------------------------------- planted mistakes

def test_planted_wrong_triangle_is_caught(monkeypatch):
    monkeypatch.setattr(o1, "triangle", lambda k: [(i, j) for i in range(1, k + 1) for j in range(1, k - i + 1)])
    rng = np.random.default_rng(4)
    n = 16
    B = (0.5 + 0.5 * rng.random((n, 5)))
    assert not np.array_equal(o1.dgemm(np.eye(n), B, 8, "rn"), B)


def test_planted_grid_off_by_one_is_caught(monkeypatch):
    real = o1._round_to_grid
    monkeypatch.setattr(o1, "_round_to_grid", lambda R, g: real(R, g + 1))
    rng = np.random.default_rng(12)
    A = rng.integers(-63, 64, size=(5, 17)).astype(np.float64)
    B = rng.integers(-63, 64, size=(17, 4)).astype(np.float64)
    A[:, 0] = 63.0
    B[0, :] = 63.0
    C = o1.dgemm(A, B, 1, "rn")
    assert not np.array_equal(C, A @ B)


@pytest.mark.parametrize("variant", ["rn", "hybrid"])
def test_split_near_the_largest_double_stays_exact(variant):
    """A row whose maximum lies within one grid step of the largest double:
    its first slice rounds up to 2^(beta-1) on the grid 2^(1025 - beta), whose
    product 2^1024 is not a double.  The residual is still the exact
    difference (RN split, step 7), so slices and residual reconstruct the row
    exactly, and the product with a small B column stays finite."""
    big = np.nextafter(np.inf, 0.0)  # (2 - 2^-52) 2^1023
    X = np.array([[big, -big * 0.75, 1.0, 3.0e-300, 5e-324, 0.0],
                  [1.9921875 * 2.0**1023, 2.0**1000, -1.0, 0.0, 0.0, 0.0]])
    beta, k = 7, 8
    if variant == "rn":
        sl, ge, bad = o1.split_rn(X, k, beta)
        grids = ge
    else:
        sl, g0, bad = o1.split_hybrid(X, k, beta)
        grids = np.stack([g0 - beta * p for p in range(k)])
    assert not bad.any()
    assert int(grids[0, 0]) == 1025 - beta and int(sl[0, 0, 0]) == 2 ** (beta - 1)
    for i in range(X.shape[0]):
        for j in range(X.shape[1]):
            rec = sum(Fraction(int(sl[p, i, j])) * Fraction(2) ** int(grids[p, i]) for p in range(k))
            err = Fraction(float(X[i, j])) - rec
            assert abs(err) <= Fraction(2) ** int(grids[k - 1, i]) / 2, (i, j)
    B = np.zeros((6, 2))
    B[0, 0], B[1, 0], B[2, 1] = 2.0**-30, 2.0**-31, 1.0
    C = (o1.dgemm_rn if variant == "rn" else o1.dgemm_hybrid)(X, B, k)
    assert np.all(np.isfinite(C))
    exact = Fraction(float(X[0, 0])) * Fraction(2) ** -30 + Fraction(float(X[0, 1])) * Fraction(2) ** -31
    assert abs(Fraction(float(C[0, 0])) - exact) <= abs(exact) * Fraction(2) ** -40
