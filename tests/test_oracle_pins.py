"""Pins of the Ozaki Scheme II oracle to facts outside the oracle itself.

Each test checks one oracle function against something the pages or plain
mathematics fix: brute force in exact Python integers or ``fractions``, a
closed-form bound, an IEEE rounding fact, an invariant of the method, or a
number printed on a page (``tests/golden/ozaki_page_facts.json``).  The last
group plants mistakes in copies of oracle functions and checks that the pins
catch them.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import ozaki2 as oz
from fp64_gemm_emulation_ozii_amd.synthetic import hpl_like, integer_valued

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "ozaki_page_facts.json")
FACTS = json.load(open(GOLDEN))


# ----------------------------------------------------------------------------
# helpers written independently of the oracle
# ----------------------------------------------------------------------------

def int_smod(x: int, m: int) -> int:
    """Symmetric residue via Python's floor-mod: ((x + floor(m/2)) mod m) - floor(m/2)."""
    h = m // 2
    return (x + h) % m - h


def exact_matmul_int(A, B):
    m, q = len(A), len(A[0])
    n = len(B[0])
    return [[sum(int(A[i][l]) * int(B[l][j]) for l in range(q)) for j in range(n)] for i in range(m)]


def exact_ab(A, B, i, j) -> Fraction:
    return sum((Fraction(float(a)) * Fraction(float(b)) for a, b in zip(A[i, :], B[:, j])), Fraction(0))


# ----------------------------------------------------------------------------
# moduli, CRT constants, k
# ----------------------------------------------------------------------------

def moduli_ok(mods):
    if any(not (FACTS["int8_residue_range"]["modulus_min"] <= m <= FACTS["int8_residue_range"]["modulus_max"]) for m in mods):
        return False
    return all(math.gcd(a, b) == 1 for i, a in enumerate(mods) for b in mods[i + 1:])


@pytest.mark.parametrize("s", range(1, 21))
def test_moduli_pairwise_coprime_in_range(s):
    mods = oz.greedy_moduli(s)
    assert len(mods) == s and moduli_ok(mods)
    assert mods == sorted(mods, reverse=True)


def test_moduli_greedy_is_maximal():
    mods = oz.greedy_moduli(20)
    for c in range(mods[-1], 257):
        if c in mods:
            continue
        larger = [m for m in mods if m > c]
        assert any(math.gcd(c, m) > 1 for m in larger), c


def crt_roundtrip_ok(mods, combine):
    """Every X in (-M/2, M/2) is recovered from its non-negative residues."""
    M = 1
    for m in mods:
        M *= m
    xs = np.arange(-(M // 2) + (1 if M % 2 == 0 else 0), M // 2 + (0 if M % 2 == 0 else 1))
    r = [np.array([x % m for x in xs.tolist()], dtype=np.uint8) for m in mods]
    X = combine(r, mods)
    return all(int(a) == int(b) for a, b in zip(X, xs))


@pytest.mark.parametrize("mods", [[256], [4, 9, 5, 7], [256, 255], [5, 7, 11, 13]])
def test_crt_brute_force_roundtrip(mods):
    assert crt_roundtrip_ok(mods, oz.crt_combine)


@pytest.mark.parametrize("s", [1, 2, 8, 14, 18, 20])
def test_crt_weights_are_idempotents(s):
    mods = oz.greedy_moduli(s)
    M, Mt, yt = oz.crt_constants(mods)
    for t, (Mt_t, yt_t) in enumerate(zip(Mt, yt)):
        W = Mt_t * yt_t
        for u, m in enumerate(mods):
            assert W % m == (1 if u == t else 0)


def test_log2M_linear_in_s():
    """Ozaki II notes §16: M ~ m_s^s, so s log2(min m) <= log2 M <= s log2(max m)."""
    for s in range(1, 21):
        mods = oz.greedy_moduli(s)
        M, _, _ = oz.crt_constants(mods)
        assert s * math.log2(min(mods)) <= math.log2(M) <= s * math.log2(max(mods)) + 1e-9


def kbits_ok(M, q, k):
    """q 2^(2k) <= M/2 - 1 < q 2^(2k+2): the bound of Ozaki II notes §5 holds and k is the largest such."""
    return 2 * q * (1 << (2 * k)) <= M - 2 < 2 * q * (1 << (2 * k + 2))


@pytest.mark.parametrize("s", range(3, 21))
@pytest.mark.parametrize("q", [1, 2, 3, 63, 64, 65, 1000, 1024, 4096, 8192, 16384, 65536, 2**17 - 1])
def test_kbits_bound_and_maximal(s, q):
    M, _, _ = oz.crt_constants(oz.greedy_moduli(s))
    k = oz.kbits(M, q)
    if k >= 0:
        assert kbits_ok(M, q, k)
        # and the product bound that uniqueness needs: 2 * q (2^k - 1)^2 < M
        assert 2 * q * ((1 << k) - 1) ** 2 < M


def test_kbits_hand_values():
    # M = 256, q = 1: (128 - 1)/1 = 127, floor(log2 127) = 6, k = 3
    assert oz.kbits(256, 1) == 3
    # M = 256, q = 64: 127/64 -> floor(log2) = 0, k = 0 (no usable bits)
    assert oz.kbits(256, 64) == 0
    # M = 256, q = 128: 127/128 < 1 -> negative
    assert oz.kbits(256, 128) < 0


def test_kbits_monotone_in_s():
    """More moduli -> larger M -> at least as many bits (Ozaki II notes §5)."""
    for q in (64, 1024, 8192, 65536):
        ks = [oz.kbits(oz.crt_constants(oz.greedy_moduli(s))[0], q) for s in range(2, 21)]
        assert all(a <= b for a, b in zip(ks, ks[1:]))


# ----------------------------------------------------------------------------
# exponents and truncation
# ----------------------------------------------------------------------------

def special_matrix():
    rng = np.random.default_rng(7)
    A = rng.standard_normal((10, 9)) * np.exp(6 * rng.standard_normal((10, 9)))
    A[0, :] = 0.0
    A[1, :] = 5e-324            # smallest subnormal
    A[1, 3] = -2.5e-320
    A[2, :] = 0.25              # exact power of two max
    A[2, 4] = -0.5
    A[3, 2] = np.inf
    A[4, 5] = np.nan
    A[5, :] = 1.7976931348623157e308
    A[6, 0] = -(2.0 ** -1022)   # smallest normal
    A[6, 1:] = 0.0
    A[7, :] = -1.0
    return A


def exponent_ok(row, e):
    vals = [abs(float(v)) for v in row]
    if any(not math.isfinite(v) for v in vals):
        return e == oz.NONFINITE
    mx = max(vals) if vals else 0.0
    if mx == 0.0:
        return e == 0
    return Fraction(2) ** (e - 1) <= Fraction(mx) < Fraction(2) ** e


def test_row_exponents_bracket_the_row_max():
    A = special_matrix()
    e = oz.row_exponents(A)
    assert e.dtype == np.int32
    for i in range(A.shape[0]):
        assert exponent_ok(A[i, :], int(e[i])), i


def test_col_exponents_are_row_exponents_of_transpose():
    A = special_matrix()
    f = oz.col_exponents(A.T.copy())
    for j in range(A.shape[0]):
        assert exponent_ok(A[j, :], int(f[j]))


def trunc_ok(A, e, k, Ap):
    for i in range(A.shape[0]):
        for l in range(A.shape[1]):
            if int(e[i]) == oz.NONFINITE:
                if Ap[i, l] != 0:
                    return False
                continue
            want = int(Fraction(float(A[i, l])) * Fraction(2) ** (k - int(e[i])))   # int() truncates toward 0
            if Fraction(float(Ap[i, l])) != want or abs(want) > (1 << k) - 1:
                return False
    return True


@pytest.mark.parametrize("k", [1, 7, 26, 48, 51, 53, 59, 64, 66])
def test_truncation_matches_exact_rational(k):
    A = special_matrix()
    e = oz.row_exponents(A)
    Ap = oz.truncate_rows(A, e, k)
    assert trunc_ok(A, e, k, Ap)
    assert not np.any(np.signbit(Ap) & (Ap == 0))


def test_truncation_keeps_k_bits_of_row_max():
    A, _ = hpl_like(16, 40, 1, 1.0, seed=3)
    k = 48
    e = oz.row_exponents(A)
    Ap = oz.truncate_rows(A, e, k)
    assert np.all(np.max(np.abs(Ap), axis=1) >= 2.0 ** (k - 1))
    assert np.all(np.max(np.abs(Ap), axis=1) <= 2.0 ** k - 1)


# ----------------------------------------------------------------------------
# residues, products, re-reduction
# ----------------------------------------------------------------------------

def test_smod_matches_integer_definition():
    rng = np.random.default_rng(11)
    vals = [0, 1, -1, 127, 128, -128, -129, 255, 256, -256, 2**53 - 1, -(2**53 - 1), 2**60, -(2**66 - 2**13)]
    vals += [int(v) for v in rng.integers(-(2**52), 2**52, size=300)]
    # large integers with trailing zero bits (exact doubles up to 2^66)
    vals += [int(v) << int(sh) for v, sh in zip(rng.integers(-(2**52), 2**52, size=100), rng.integers(1, 14, size=100))]
    X = np.array(vals, dtype=np.float64)
    assert all(int(x) == v for x, v in zip(X, vals))
    for m in oz.greedy_moduli(20) + [2, 3, 4]:
        r = oz.smod(X, m)
        assert r.dtype == np.int8
        assert [int(v) for v in r] == [int_smod(v, m) for v in vals], m


def test_smod_range_for_256_is_page_range():
    facts = FACTS["int8_residue_range"]
    r = oz.smod(np.arange(-1000, 1000, dtype=np.float64), 256)
    assert int(r.min()) == facts["residue_min"] and int(r.max()) == facts["residue_max"]


def product_ok(At, Bt, C):
    return np.array_equal(np.array(exact_matmul_int(At.tolist(), Bt.tolist()), dtype=np.int64), C.astype(np.int64))


def test_residue_product_brute_force():
    rng = np.random.default_rng(5)
    At = rng.integers(-128, 128, size=(7, 131)).astype(np.int8)
    Bt = rng.integers(-128, 128, size=(131, 5)).astype(np.int8)
    At[0, :] = -128
    Bt[:, 0] = -128
    C = oz.residue_product(At, Bt)
    assert C.dtype == np.int64
    assert product_ok(At, Bt, C)


def test_residue_product_worst_case_fits_int32():
    facts = FACTS["int32_exact_dot"]
    q = 2 ** facts["q_limit_log2"] - 1
    At = np.full((1, q), -128, dtype=np.int8)
    Bt = np.full((q, 1), -128, dtype=np.int8)
    C = oz.residue_product(At, Bt)
    assert int(C[0, 0]) == q * 2 ** facts["product_bound_log2"] < 2**31
    # one past the int32 limit: the product leaves int32 and is still exact
    At = np.full((1, q + 2), -128, dtype=np.int8)
    Bt = np.full((q + 2, 1), -128, dtype=np.int8)
    assert int(oz.residue_product(At, Bt)[0, 0]) == (q + 2) * 2**14 > 2**31 - 1


def test_long_inner_dimension_brute_force():
    """q > 2^17 (K split into exact int32 blocks on the GPU): the oracle's
    result still equals the exact rational product rounded once."""
    rng = np.random.default_rng(77)
    q = 2**17 + 300
    A = (rng.random((3, q)) - 0.5) * np.exp(0.5 * rng.standard_normal((3, q)))
    B = (rng.random((q, 2)) - 0.5) * np.exp(0.5 * rng.standard_normal((q, 2)))
    C, st = oz.dgemm(A, B, 14, stages=True)
    k = st["k"]
    assert k == oz.kbits(st["M"], q) >= 1
    to_int = np.vectorize(int, otypes=[object])
    X = to_int(st["Ap"]).dot(to_int(st["Bp"]))
    assert np.array_equal(st["X"], X)
    for i in range(3):
        for j in range(2):
            assert C[i, j] == oz.round_scaled(int(X[i, j]), int(st["e"][i]) + int(st["f"][j]) - 2 * k)


def test_reduce_product_nonnegative():
    C = np.array([-(2**31) + 1, -257, -1, 0, 1, 255, 256, 2**31 - 1], dtype=np.int32)
    for m in (256, 255, 253, 173):
        r = oz.reduce_product(C, m)
        assert r.dtype == np.uint8
        assert [int(v) for v in r] == [int(c) % m for c in C.tolist()]


# ----------------------------------------------------------------------------
# whole scheme: the CRT recovers the exact integer product A'B'
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("s,phi,shape", [(14, 0.5, (6, 64, 5)), (8, 1.0, (4, 33, 7)), (18, 0.5, (5, 64, 4)),
                                         (16, 4.0, (3, 100, 3)), (20, 0.0, (2, 17, 3))])
def test_crt_equals_exact_integer_product(s, phi, shape):
    m, q, n = shape
    A, B = hpl_like(m, q, n, phi, seed=s)
    C, st = oz.dgemm(A, B, s, stages=True)
    Ap = [[int(v) for v in row] for row in st["Ap"]]
    Bp = [[int(v) for v in row] for row in st["Bp"]]
    X = exact_matmul_int(Ap, Bp)
    M = st["M"]
    for i in range(m):
        for j in range(n):
            assert int(st["X"][i, j]) == X[i][j]
            assert 2 * abs(X[i][j]) < M
            for t, mt in enumerate(st["moduli"]):
                assert (X[i][j] - int(st["Ct"][t, i, j])) % mt == 0
                assert int(st["rt"][t, i, j]) == X[i][j] % mt
    # every residue plane is the symmetric residue of the integer matrix
    for t, mt in enumerate(st["moduli"]):
        assert all(int(st["Ares"][t, i, l]) == int_smod(Ap[i][l], mt) for i in range(m) for l in range(q))


# ----------------------------------------------------------------------------
# unscaling: IEEE rounding facts
# ----------------------------------------------------------------------------

TINY = 5e-324          # 2^-1074
MAXD = 1.7976931348623157e308


@pytest.mark.parametrize("X,p,want", [
    (3, 0, 3.0), (-5, 3, -40.0), (1, -1074, TINY), (1, -1075, 0.0), (3, -1075, 2 * TINY),
    (5, -1076, TINY), (7, -1076, 2 * TINY), (2**53 + 1, 0, 2.0**53), (2**53 + 3, 0, 2.0**53 + 4),
    (2**53 - 1, 971, MAXD), (2**54 - 1, 970, math.inf), (-1, 1024, -math.inf),
    ((2**53 - 1) * 2 + 1, 970, math.inf), (2**52 * 3 + 1, -1076 - 52, 2.0**-1074 * 1),
])
def test_round_scaled_ieee_cases(X, p, want):
    got = oz.round_scaled(X, p)
    assert got == want and math.copysign(1, got) == math.copysign(1, want)


def test_round_scaled_negative_underflow_keeps_sign():
    assert math.copysign(1, oz.round_scaled(-1, -1076)) == -1.0


def test_round_scaled_matches_ldexp_when_exact():
    rng = np.random.default_rng(3)
    for X, p in zip(rng.integers(-(2**53) + 1, 2**53, size=200), rng.integers(-1000, 900, size=200)):
        assert oz.round_scaled(int(X), int(p)) == math.ldexp(float(int(X)), int(p))


# ----------------------------------------------------------------------------
# special cases with known answers
# ----------------------------------------------------------------------------

def test_integer_inputs_are_exact():
    """|entries| <= 2^10, q = 64, s = 14 (k = 51): no truncation, C == A B exactly."""
    A, B = integer_valued(9, 64, 7, 2**10, seed=1)
    C = oz.dgemm(A, B, 14)
    want = exact_matmul_int(A.astype(np.int64).tolist(), B.astype(np.int64).tolist())
    assert [[float(v) for v in row] for row in want] == C.tolist()


def test_identity_is_exact_with_enough_bits():
    """Entries in [1/4, 1/2) times I: A' is exact once k >= 53 (s = 16, q = 64 -> k = 59)."""
    rng = np.random.default_rng(2)
    A = 0.25 + 0.25 * rng.random((12, 64))
    C = oz.dgemm(A, np.eye(64), 16)
    assert np.array_equal(C, A)


def test_zero_matrix_gives_positive_zero():
    C = oz.dgemm(np.zeros((4, 8)), np.ones((8, 3)), 14)
    assert np.all(C == 0) and not np.any(np.signbit(C))


def test_nonfinite_rows_and_columns_become_nan():
    A, B = hpl_like(5, 16, 4, 0.5, seed=9)
    A[2, 7] = np.inf
    B[3, 1] = np.nan
    C = oz.dgemm(A, B, 14)
    assert np.all(np.isnan(C[2, :])) and np.all(np.isnan(C[:, 1]))
    mask = np.ones_like(C, dtype=bool)
    mask[2, :] = False
    mask[:, 1] = False
    assert np.all(np.isfinite(C[mask]))


@pytest.mark.parametrize("s", [8, 10, 14, 16])
def test_error_bound_against_exact_product(s):
    """|C - AB| <= 2^(e_i-k) sum|b_lj| + 2^(f_j-k) sum|a_il| + q 2^(e_i+f_j-2k) + 2^-53 |C|,
    the bound implied by |a - A'/D| < 2^(e_i - k) (truncation is the only error, Ozaki II notes §6)."""
    A, B = hpl_like(5, 48, 6, 1.0, seed=4)
    C, st = oz.dgemm(A, B, s, stages=True)
    k = st["k"]
    for i in range(5):
        for j in range(6):
            ei, fj = int(st["e"][i]), int(st["f"][j])
            bound = (Fraction(2) ** (ei - k) * sum(Fraction(abs(float(b))) for b in B[:, j])
                     + Fraction(2) ** (fj - k) * sum(Fraction(abs(float(a))) for a in A[i, :])
                     + 48 * Fraction(2) ** (ei + fj - 2 * k)
                     + Fraction(2) ** -53 * abs(Fraction(float(C[i, j]))))
            assert abs(Fraction(float(C[i, j])) - exact_ab(A, B, i, j)) <= bound


def test_accuracy_grows_with_moduli():
    A, B = hpl_like(4, 256, 4, 0.5, seed=0)
    rows = [0, 1, 2, 3] * 4
    cols = [c for c in range(4) for _ in range(4)]
    bits = {s: oz.correct_bits(oz.dgemm(A, B, s), A, B, rows, cols) for s in (8, 12, 16)}
    assert bits[8] + 10 < bits[12] and bits[12] + 10 < bits[16]


# ----------------------------------------------------------------------------
# invariants
# ----------------------------------------------------------------------------

def test_power_of_two_scaling_negation_transpose_permutation():
    A, B = hpl_like(7, 40, 6, 1.0, seed=8)
    C = oz.dgemm(A, B, 14)
    assert np.array_equal(oz.dgemm(A * 2.0**37, B, 14), C * 2.0**37)
    assert np.array_equal(oz.dgemm(A, B * 2.0**-60, 14), C * 2.0**-60)
    assert np.array_equal(oz.dgemm(-A, B, 14), -C)
    assert np.array_equal(oz.dgemm(B.T.copy(), A.T.copy(), 14), C.T)
    pr = np.random.default_rng(1).permutation(7)
    pc = np.random.default_rng(2).permutation(6)
    assert np.array_equal(oz.dgemm(A[pr], B[:, pc], 14), C[pr][:, pc])


def test_block_entries_equal_full_entries():
    A, B = hpl_like(20, 50, 18, 0.5, seed=6)
    C = oz.dgemm(A, B, 13)
    rows, cols = [3, 0, 19], [17, 2]
    assert np.array_equal(oz.dgemm_block(A, B, 13, rows, cols), C[np.ix_(rows, cols)])


# ----------------------------------------------------------------------------
# planted mistakes: each pin above must reject a plausible bug
# ----------------------------------------------------------------------------

def _crt_without_inverse(r, moduli):
    M, Mt, _ = oz.crt_constants(moduli)
    Z = sum(np.asarray(rt, np.int64).astype(object) * Mt_t for rt, Mt_t in zip(r, Mt))
    X = Z % M
    return np.where(X > M // 2, X - M, X)


def _crt_without_symmetric(r, moduli):
    M, Mt, yt = oz.crt_constants(moduli)
    Z = sum(np.asarray(rt, np.int64).astype(object) * (a * b) for rt, a, b in zip(r, Mt, yt))
    return Z % M


def test_planted_crt_mistakes_are_caught():
    for mods in ([4, 9, 5, 7], [256, 255]):
        assert not crt_roundtrip_ok(mods, _crt_without_inverse)
        assert not crt_roundtrip_ok(mods, _crt_without_symmetric)


def test_planted_kbits_mistakes_are_caught():
    M, _, _ = oz.crt_constants(oz.greedy_moduli(14))
    k = oz.kbits(M, 8192)
    assert not kbits_ok(M, 8192, k + 1) and not kbits_ok(M, 8192, k - 1)
    # using log2(M/2/q) without the -1 and with ceil would give k + 1 for some q
    bad = [q for q in range(1, 2000) if math.ceil(0.5 * math.log2(M / 2 / q)) != oz.kbits(M, q)]
    assert bad


def test_planted_truncation_mistakes_are_caught():
    A = special_matrix()
    e = oz.row_exponents(A)
    k = 48
    assert not trunc_ok(A, e, k, np.round(np.ldexp(A, (k - np.where(e == oz.NONFINITE, 0, e)).astype(np.int32)[:, None])))
    wrong_e = np.where(e == oz.NONFINITE, e, e - 1).astype(np.int32)       # ceil-vs-frexp slip
    assert not all(exponent_ok(A[i, :], int(wrong_e[i])) for i in range(A.shape[0]))


def test_planted_product_mistakes_are_caught():
    rng = np.random.default_rng(5)
    At = rng.integers(-128, 128, size=(6, 6)).astype(np.int8)
    Bt = rng.integers(-128, 128, size=(6, 6)).astype(np.int8)
    assert not product_ok(At, Bt, oz.residue_product(At, Bt.T.copy()))      # transposed operand
    assert not product_ok(At, Bt, (At.astype(np.int32) @ Bt.astype(np.int32)).astype(np.int8).astype(np.int32))


def test_planted_smod_mistake_is_caught():
    X = np.arange(-600, 600, dtype=np.float64)
    wrong = np.fmod(X, 255.0).astype(np.int8)           # plain fmod is not symmetric
    assert [int(v) for v in wrong] != [int_smod(int(v), 255) for v in X]


def test_scheme1_count_table_from_page():
    """The notes' slice-count table is k(k+1)/2 (Ozaki II notes §2)."""
    table = FACTS["scheme1_gemm_count"]["slices_to_gemms"]
    for k, count in table.items():
        k = int(k)
        assert sum(1 for i in range(1, k + 1) for j in range(1, k + 1) if i + j <= k + 1) == count


# ------------------------------------------------------------------ OS II-fast

def _frac_sq_norm(v):
    return sum(Fraction(float(x)) ** 2 for x in v)


@pytest.mark.parametrize("s", [1, 2, 5, 8, 14, 16, 20])
def test_fast_budget_splits_floor_log2_half_m(s):
    M, _, _ = oz.crt_constants(oz.greedy_moduli(s))
    kA, kB = oz.cs_budget(M)
    assert kB - kA in (0, 1)
    assert 2 ** (kA + kB) <= M // 2 - 1 < 2 ** (kA + kB + 1)


def test_norm_units_bound_the_squared_norm_tightly():
    rng = np.random.default_rng(31)
    A = (rng.random((7, 300)) - 0.5) * np.exp(2 * rng.standard_normal((7, 300)))
    A[2, :] = 0.0
    A[3, 4] = 2.0**-1070
    e = oz.row_exponents(A)
    S = oz.row_norm_units(A, e)
    for i in range(A.shape[0]):
        exact = _frac_sq_norm(A[i] * 2.0 ** -int(e[i])) if A[i].any() else Fraction(0)
        bound = Fraction(S[i], 2 ** (2 * oz.NORM_GRID))
        assert bound >= exact
        # each entry is rounded up by less than 2^-20 (relative to 2^e)
        slack = sum(2 * abs(Fraction(float(x)) * Fraction(2) ** -int(e[i])) * Fraction(1, 2**20) + Fraction(1, 2**40)
                    for x in A[i])
        assert bound - exact <= slack


@pytest.mark.parametrize("s,q", [(6, 40), (10, 64), (14, 100), (18, 33)])
def test_fast_bound_keeps_crt_exact(s, q):
    """OS II-fast: ||A'_i|| <= 2^kappa_A, ||B'_j|| <= 2^kappa_B, hence by
    Cauchy-Schwarz |(A'B')_ij| < M/2 and the CRT returns A'B' exactly."""
    rng = np.random.default_rng(s * 100 + q)
    A = (rng.random((9, q)) - 0.5) * np.exp(rng.standard_normal((9, q)))
    B = (rng.random((q, 8)) - 0.5) * np.exp(rng.standard_normal((q, 8)))
    A[0, :] = 1.0  # flat row: the bound is nearly tight
    C, st = oz.dgemm(A, B, s, stages=True, bound="fast")
    M = st["M"]
    kA, kB = oz.cs_budget(M)
    to_int = np.vectorize(int, otypes=[object])
    Ap = to_int(st["Ap"])
    Bp = to_int(st["Bp"])
    for i in range(A.shape[0]):
        assert sum(int(x) ** 2 for x in Ap[i]) <= 4 ** kA
    for j in range(B.shape[1]):
        assert sum(int(x) ** 2 for x in Bp[:, j]) <= 4 ** kB
    exact = Ap.dot(Bp)
    assert np.array_equal(st["X"], exact)
    assert all(2 * abs(int(v)) < M for v in exact.flat)


def test_fast_bound_tight_case_and_planted_overshoot(monkeypatch):
    """All-ones rows with q = 4^j meet the bound with equality; a budget one
    bit larger on each side breaks the CRT uniqueness."""
    s, q = 9, 64
    A = np.ones((3, q))
    B = np.ones((q, 2))
    C, st = oz.dgemm(A, B, s, stages=True, bound="fast")
    kA, kB = oz.cs_budget(st["M"])
    assert int(st["X"][0, 0]) == 2 ** (kA + kB)
    assert np.all(C == q)
    real = oz.cs_budget
    monkeypatch.setattr(oz, "cs_budget", lambda M: tuple(v + 1 for v in real(M)))
    C2, st2 = oz.dgemm(A, B, s, stages=True, bound="fast")
    to_int = np.vectorize(int, otypes=[object])
    exact = to_int(st2["Ap"]).dot(to_int(st2["Bp"]))
    assert not np.array_equal(st2["X"], exact)


def test_fast_bound_gains_bits_on_wide_rows():
    rng = np.random.default_rng(8)
    q = 256
    A = (rng.random((6, q)) - 0.5) * np.exp(rng.standard_normal((6, q)))
    B = (rng.random((q, 6)) - 0.5) * np.exp(rng.standard_normal((q, 6)))
    rows, cols = np.arange(6).repeat(6), np.tile(np.arange(6), 6)
    for s in (8, 10, 12):
        cons = oz.correct_bits(oz.dgemm(A, B, s), A, B, rows, cols)
        fast = oz.correct_bits(oz.dgemm(A, B, s, bound="fast"), A, B, rows, cols)
        assert fast >= cons + 2.0, (s, cons, fast)


def test_fast_bound_special_rows():
    rng = np.random.default_rng(6)
    A = rng.standard_normal((5, 20))
    B = rng.standard_normal((20, 4))
    A[1, :] = 0.0
    A[2, 3] = np.nan
    B[:, 1] = 0.0
    C = oz.dgemm(A, B, 12, bound="fast")
    assert np.all(C[1, :] == 0.0) and np.all(np.isnan(C[2, :]))
    assert np.all(C[[0, 3, 4]][:, 1] == 0.0)
    Ci = oz.dgemm(np.round(A * 8), np.round(B * 8), 12, bound="fast")
    ref = np.round(A * 8) @ np.round(B * 8)
    ok = ~np.isnan(Ci)
    assert np.array_equal(Ci[ok], ref[ok])


def test_tiled_oracle_pool_equals_the_whole_oracle():
    """The process-pool evaluation used for full-size parity (tests/oracle_pool.py)
    reassembles exactly the whole oracle result, ragged tiles included."""
    from oracle_pool import oracle_full
    from fp64_gemm_emulation_ozii_amd.synthetic import hpl_like
    m, q, n = 37, 150, 29
    A, B = hpl_like(m, q, n, 1.0, seed=5)
    whole = oz.dgemm(A, B, 14)
    tiled = oracle_full(m, q, n, 1.0, 5, 14, tiles=(3, 2), workers=2, timeout=300)
    assert np.array_equal(whole.view(np.uint64), tiled.view(np.uint64))


# ---------------------------------------------------------------- OS II-accu

def _frac_x(v: float, e: int) -> Fraction:
    return abs(Fraction(float(v))) / Fraction(2) ** int(e)


def _accu_inputs(seed=0, m=9, q=150, n=8, phi=2.0):
    rng = np.random.default_rng(seed)
    A = (rng.random((m, q)) - 0.5) * np.exp(phi * rng.standard_normal((m, q)))
    B = (rng.random((q, n)) - 0.5) * np.exp(phi * rng.standard_normal((q, n)))
    A[0, :] = 0.0                               # zero row
    A[1, :] = np.ldexp(1.0, -(np.arange(q) // 2))  # powers of two on both sides of the band edge
    A[2, :] = 2.0**-1074                        # smallest subnormals
    A[3, 5] = 2.0**-1060                        # a subnormal in a normal row
    B[:, 0] = 1.0                               # flat column: the bound is nearly tight
    B[:, 1] = 0.0
    B[7, 2] = np.nan
    return A, B


def test_accu_bands_round_up_exactly():
    """H/127 + Lo/(127 2^7) >= x = |a| 2^-e, with H = ceil(127 x) on
    x >= 2^-7 and Lo = ceil(127 2^7 x) below: checked with exact rationals,
    band edges, subnormals and Inf/NaN rows included."""
    A, _ = _accu_inputs()
    A[4, 3] = np.inf
    e = oz.row_exponents(A).astype(np.int64)
    H, Lo = oz.accu_bands(A, e)
    for r in range(A.shape[0]):
        for l in range(A.shape[1]):
            if e[r] == oz.NONFINITE:
                assert H[r, l] == 0 and Lo[r, l] == 0
                continue
            x = _frac_x(A[r, l], e[r])
            assert 0 <= x < 1
            if x == 0:
                assert H[r, l] == 0 and Lo[r, l] == 0
            elif x >= Fraction(1, 128):
                assert Lo[r, l] == 0 and H[r, l] == math.ceil(127 * x)
            else:
                assert H[r, l] == 0 and Lo[r, l] == math.ceil(127 * 128 * x)
            assert 0 <= H[r, l] <= 127 and 0 <= Lo[r, l] <= 127


def _check_bound_holds(A, B, N=None, L=None):
    """sum_l x_il y_lj <= N_ij / ACCU_DEN (when N is given) and <= 2^L_ij
    (when L is given; L = -128 means the sum is 0), exactly."""
    e = oz.row_exponents(A).astype(np.int64)
    f = oz.col_exponents(B).astype(np.int64)
    for i in range(A.shape[0]):
        if e[i] == oz.NONFINITE:
            continue
        x = [_frac_x(v, e[i]) for v in A[i]]
        for j in range(B.shape[1]):
            if f[j] == oz.NONFINITE:
                continue
            exact = sum(xi * _frac_x(v, f[j]) for xi, v in zip(x, B[:, j]))
            if N is not None:
                assert exact <= Fraction(int(N[i, j]), oz.ACCU_DEN), (i, j)
            if L is not None:
                if L[i, j] == oz.ACCU_LZERO:
                    assert exact == 0, (i, j)
                else:
                    assert exact <= Fraction(2) ** int(L[i, j]), (i, j, float(exact), int(L[i, j]))


@pytest.mark.parametrize("seed,phi", [(0, 2.0), (1, 0.5), (2, 6.0)])
def test_accu_bound_is_an_upper_bound(seed, phi):
    """The two-band int8 bound of OS II-accu never falls below the exact
    sum_l x_il y_lj, and L_ij is the ceiling of its log2."""
    A, B = _accu_inputs(seed, phi=phi)
    e = oz.row_exponents(A).astype(np.int64)
    f = oz.col_exponents(B).astype(np.int64)
    N = oz.accu_bound(A, B, e, f)
    L = oz.accu_bound_exponents(A, B, e, f)
    _check_bound_holds(A, B, N, L)
    assert np.all(L[0, :] == oz.ACCU_LZERO) and np.all(L[:, 1] == oz.ACCU_LZERO)
    # N written out from the bands for a few entries; L is the ceiling of log2
    Ha, La = oz.accu_bands(A, e)
    Hb, Lb = oz.accu_bands(B.T, f)
    for i, j in [(3, 0), (5, 3), (1, 4), (2, 0)]:
        Nij = (int(Ha[i] @ Hb[j]) << 14) + ((int(Ha[i] @ Lb[j]) + int(La[i] @ Hb[j])) << 7) \
            + 127 * min(int(La[i].sum()), int(Lb[j].sum()))
        assert Nij == N[i, j]
        bound = Fraction(Nij, 127 * 127 * 2**14)
        assert Fraction(2) ** int(L[i, j] - 1) < bound <= Fraction(2) ** int(L[i, j])


def test_accu_bound_is_close_to_the_exact_sum():
    """On log-normal rows (phi = 1) the bound stays within a factor 4 of the
    exact sum for every entry and within 2 for most: the bands keep about
    seven bits of each magnitude over fourteen bits of range."""
    A, B = hpl_like(12, 400, 10, 1.0, seed=4)
    e = oz.row_exponents(A).astype(np.int64)
    f = oz.col_exponents(B).astype(np.int64)
    L = oz.accu_bound_exponents(A, B, e, f)
    x = np.ldexp(np.abs(A), -e[:, None])
    y = np.ldexp(np.abs(B), -f[None, :])
    ratio = np.exp2(L) / (x @ y)
    assert np.all(ratio >= 1.0 - 1e-12) and np.all(ratio <= 4.0) and np.median(ratio) <= 2.0


def test_accu_planted_underestimates_are_caught(monkeypatch):
    """Rounding the bands down, or dropping the low band of B (the HL and LL
    terms), gives bounds below the exact sum, which the upper-bound check
    detects: on all-ones rows the high band is within 1% of exact, and a
    row whose maximum meets only low-band entries of the column needs HL."""
    q = 64
    A1, B1 = np.ones((2, q)), np.ones((q, 2))          # x = y = 1/2: 127 x = 63.5
    A2 = np.full((1, q), 2.0**-20)
    B2 = np.full((q, 1), 2.0**-20)
    A2[0, 0], A2[0, 5] = 1.0, 0.0                      # A's maximum meets B's low band
    B2[5, 0] = 1.0                                     # B's maximum meets a zero of A
    real = oz.accu_bands
    cases = []
    for A, B in [(A1, B1), (A2, B2)]:
        e = oz.row_exponents(A).astype(np.int64)
        f = oz.col_exponents(B).astype(np.int64)
        _check_bound_holds(A, B, N=oz.accu_bound(A, B, e, f))
        cases.append((A, B, e, f))

    def floor_bands(X, ex):
        H, Lo = real(X, ex)
        return np.maximum(H - 1, 0), np.maximum(Lo - 1, 0)

    monkeypatch.setattr(oz, "accu_bands", floor_bands)
    A, B, e, f = cases[0]
    with pytest.raises(AssertionError):
        _check_bound_holds(A, B, N=oz.accu_bound(A, B, e, f))

    def no_low_band_of_b(X, ex):
        H, Lo = real(X, ex)
        return (H, 0 * Lo) if X.shape == B2.T.shape and np.array_equal(X, B2.T) else (H, Lo)

    monkeypatch.setattr(oz, "accu_bands", no_low_band_of_b)
    A, B, e, f = cases[1]
    with pytest.raises(AssertionError):
        _check_bound_holds(A, B, N=oz.accu_bound(A, B, e, f))


@pytest.mark.parametrize("s", [8, 12, 14, 17])
def test_accu_scaling_is_feasible_and_tight(s):
    """a_i + b_j + L_ij <= K2 everywhere; every row and column meets the
    budget with equality somewhere (or sits at the cap)."""
    A, B = _accu_inputs(s, phi=2.0)
    M = oz.crt_constants(oz.greedy_moduli(s))[0]
    K2 = (M // 2 - 1).bit_length() - 1
    e = oz.row_exponents(A).astype(np.int64)
    f = oz.col_exponents(B).astype(np.int64)
    L = oz.accu_budget_exponents(A, B, e, f, M)
    a, b = oz.accu_scaling(L, K2)
    slack = K2 - (a[:, None] + b[None, :] + L)
    assert np.all(slack >= 0)
    for i in range(L.shape[0]):
        assert a[i] == oz.ACCU_KMAX or np.any(slack[i, :] == 0)
    for j in range(L.shape[1]):
        assert b[j] == oz.ACCU_KMAX or np.any(slack[:, j] == 0)


def _check_budget_exact(N, L, M):
    """With T = K2 - L: 2^T N / ACCU_DEN <= M/2 - 1 < 2^(T+1) N / ACCU_DEN
    wherever N > 0 (Python integers), and L = ACCU_LZERO where N = 0."""
    K2 = (M // 2 - 1).bit_length() - 1
    V = (M // 2 - 1) * oz.ACCU_DEN
    for (i, j), n in np.ndenumerate(N):
        if n == 0:
            assert L[i, j] == oz.ACCU_LZERO, (i, j)
            continue
        T = K2 - int(L[i, j])
        assert int(n) << T <= V, ("budget exceeded", i, j)
        assert int(n) << (T + 1) > V, ("budget not maximal", i, j)


@pytest.mark.parametrize("s", [4, 9, 14, 17, 20])
def test_accu_budget_is_exact_and_maximal(s):
    """The accu budget compares the two-band bound with M/2 - 1 exactly: the
    row and column bit counts of entry (i, j) may sum to T_ij and not one
    more.  It is never tighter than the power-of-two ceiling of the bound."""
    A, B = _accu_inputs(s, phi=2.0)
    M = oz.crt_constants(oz.greedy_moduli(s))[0]
    K2 = (M // 2 - 1).bit_length() - 1
    e = oz.row_exponents(A).astype(np.int64)
    f = oz.col_exponents(B).astype(np.int64)
    N = oz.accu_bound(A, B, e, f)
    Lb = oz.accu_budget_exponents(A, B, e, f, M)
    _check_budget_exact(N, Lb, M)
    Lc = oz.accu_bound_exponents(A, B, e, f)
    assert np.all(Lb <= Lc)
    # at least one entry gains a bit over the ceiling rule for these inputs
    assert np.any(Lb < Lc) or s == 4


def test_accu_budget_planted_mistakes_are_caught():
    """The old power-of-two ceiling (feasible, not maximal) and a budget one
    bit too wide (not feasible) both fail the exactness check."""
    A, B = _accu_inputs(3, phi=1.0)
    M = oz.crt_constants(oz.greedy_moduli(14))[0]
    e = oz.row_exponents(A).astype(np.int64)
    f = oz.col_exponents(B).astype(np.int64)
    N = oz.accu_bound(A, B, e, f)
    Lceil = oz.accu_bound_exponents(A, B, e, f)  # the budget K2 - ceil(log2(N / ACCU_DEN))
    Lb = oz.accu_budget_exponents(A, B, e, f, M)
    assert np.any(Lceil != Lb)
    with pytest.raises(AssertionError):
        _check_budget_exact(N, Lceil, M)
    wide = np.where(Lb == oz.ACCU_LZERO, Lb, Lb - 1)
    with pytest.raises(AssertionError):
        _check_budget_exact(N, wide, M)


@pytest.mark.parametrize("s,q", [(8, 40), (12, 150), (14, 200), (18, 33)])
def test_accu_keeps_crt_exact(s, q):
    """OS II-accu: |A'_i| < 2^a_i per entry, the CRT returns A'B' exactly and
    2 |A'B'| < M, with Python integers."""
    A, B = _accu_inputs(s + q, q=q, phi=1.5)
    B[7, 2] = 0.5
    C, st = oz.dgemm(A, B, s, stages=True, bound="accu")
    M, k = st["M"], st["k"]
    to_int = np.vectorize(int, otypes=[object])
    Ap, Bp = to_int(st["Ap"]), to_int(st["Bp"])
    e, f = st["e"], st["f"]
    for i in range(A.shape[0]):
        if e[i] != oz.NONFINITE:
            assert all(abs(v) < 2 ** (k - int(e[i]) + int(oz.row_exponents(A)[i])) for v in Ap[i])
    absP = np.abs(Ap).dot(np.abs(Bp))
    assert all(2 * int(v) < M for v in absP.flat)
    assert np.array_equal(st["X"], Ap.dot(Bp))


def test_accu_gains_bits_over_fast_on_wide_rows():
    A, B = hpl_like(24, 512, 24, 2.0, seed=9)
    rows, cols = np.arange(24).repeat(24), np.tile(np.arange(24), 24)
    for s in (12, 14):
        fast = oz.correct_bits(oz.dgemm(A, B, s, bound="fast"), A, B, rows, cols)
        accu = oz.correct_bits(oz.dgemm(A, B, s, bound="accu"), A, B, rows, cols)
        assert accu >= fast + 0.5, (s, fast, accu)


def test_accu_special_rows_and_integers():
    rng = np.random.default_rng(6)
    A = rng.standard_normal((5, 20))
    B = rng.standard_normal((20, 4))
    A[1, :] = 0.0
    A[2, 3] = np.nan
    B[:, 1] = 0.0
    C = oz.dgemm(A, B, 12, bound="accu")
    assert np.all(C[1, :] == 0.0) and np.all(np.isnan(C[2, :]))
    assert np.all(C[[0, 3, 4]][:, 1] == 0.0)
    Ai, Bi = integer_valued(7, 64, 5, 2**10, seed=3)
    assert np.array_equal(oz.dgemm(Ai, Bi, 14, bound="accu"), Ai @ Bi)
