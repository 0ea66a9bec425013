"""Seeded random parity sweeps of ozgemm_dgemm and ozgemm_scheme1_dgemm
against the oracles.

24 cases drawn from numpy.random.default_rng(20261202):
  * shapes m, n in 1..300 and q in 1..6000 (some long enough for K parts,
    some short enough for the eight-wavefront product form);
  * s in 6..20 where the bit budget leaves k >= 1;
  * phi in {0, 0.5, 1, 2, 8} (the HPL-like generator);
  * the conservative or the OS II-fast bit budget;
  * leading-dimension padding (padding holds NaN, which must never be read);
  * sometimes a zero row or column, a row scaled into the subnormal range or
    towards overflow, or an Inf/NaN entry.
Every C must equal the oracle's bit for bit (NaN positions alike) and, for
Scheme II, lie within 2^-50 (|A||B|)_ij of it.  The Scheme I sweep draws
16 cases of the same kinds with k in 2..10 slices and the RN or the Hybrid
variant.  12 more Scheme II cases draw q from [4000, 9000), around the range
where B's exponents are taken in its residue pass, and 10 run the OS II-accu
budget with phi up to 16.
"""
import numpy as np
import pytest

from oracle import ozaki2 as oz
from fp64_gemm_emulation_ozii_amd import ozgemm as L
from fp64_gemm_emulation_ozii_amd.synthetic import hpl_like

from gpu_util import configure, dev_colmajor, first_diff, log, run_dgemm, same_doubles, within_tolerance

pytestmark = pytest.mark.gpu

MAX_M, MAX_N, MAX_Q = 300, 300, 6000


def draw_cases(count: int, seed: int = 20261202):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < count:
        m = int(rng.integers(1, MAX_M + 1))
        n = int(rng.integers(1, MAX_N + 1))
        q = int(rng.integers(1, 600)) if rng.random() < 0.5 else int(rng.integers(600, MAX_Q + 1))
        s = int(rng.integers(6, 21))
        bound = "fast" if rng.random() < 0.35 else "conservative"
        M, _, _ = oz.crt_constants(oz.greedy_moduli(s))
        if bound == "conservative" and oz.kbits(M, q) < 1:
            continue
        if bound == "fast" and s < 8:
            continue
        phi = float(rng.choice([0.0, 0.5, 1.0, 2.0, 8.0]))
        pads = tuple(int(rng.integers(0, 4)) for _ in range(3))
        special = str(rng.choice(["none", "none", "zero", "tiny", "huge", "nonfinite"]))
        cases.append((m, n, q, s, bound, phi, pads, special, int(rng.integers(0, 2**31))))
    return cases


CASES = draw_cases(24)


@pytest.fixture(scope="module", autouse=True)
def random_config():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    configure(MAX_M, MAX_N, MAX_Q, 20)
    yield
    L.ozgemm_set_bound(L.OZGEMM_BOUND_CONSERVATIVE)
    L.ozgemm_free()


def make_inputs(m, n, q, phi, special, seed):
    A, B = hpl_like(m, q, n, phi, seed=seed)
    rng = np.random.default_rng(seed + 1)
    i, j, l = int(rng.integers(0, m)), int(rng.integers(0, n)), int(rng.integers(0, q))
    if special == "zero":
        A[i, :] = 0.0
        B[:, j] = 0.0
    elif special == "tiny":
        A[i, :] *= 2.0 ** -1000
        B[:, j] *= 2.0 ** -60
    elif special == "huge":
        A[i, :] *= 2.0 ** 900
        B[:, j] *= 2.0 ** 200
    elif special == "nonfinite":
        A[i, l] = np.inf
        B[l, j] = np.nan
    return A, B


@pytest.mark.parametrize("case", range(len(CASES)))
def test_random_case(case):
    m, n, q, s, bound, phi, pads, special, seed = CASES[case]
    log(f"random case {case}: m={m} n={n} q={q} s={s} bound={bound} phi={phi} pads={pads} special={special}")
    A, B = make_inputs(m, n, q, phi, special, seed)
    L.ozgemm_set_bound(L.OZGEMM_BOUND_FAST if bound == "fast" else L.OZGEMM_BOUND_CONSERVATIVE)
    try:
        C, _ = run_dgemm(A, B, s, lda=m + pads[0], ldb=q + pads[1], ldc=m + pads[2])
    finally:
        L.ozgemm_set_bound(L.OZGEMM_BOUND_CONSERVATIVE)
    ref = oz.dgemm(A, B, s, bound=bound)
    assert same_doubles(C, ref), first_diff(C, ref)
    with np.errstate(invalid="ignore", over="ignore"):
        finite_rows = np.isfinite(A).all(axis=1)
        finite_cols = np.isfinite(B).all(axis=0)
        sub = np.ix_(finite_rows, finite_cols)
        assert within_tolerance(C[sub], ref[sub], A[finite_rows], B[:, finite_cols])


# ---- 12 more Scheme II cases with q around the one-pass range of B ----

def draw_one_pass_cases(count: int, seed: int = 20261204):
    """q in [4000, 9000): mostly inside [OZGEMM_ONE_PASS_Q_MIN,
    OZGEMM_ONE_PASS_Q_MAX], where ozgemm_dgemm takes B's exponents in its
    residue pass, with ragged K; the rest on either side of it."""
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < count:
        m = int(rng.integers(1, MAX_M + 1))
        n = int(rng.integers(1, MAX_N + 1))
        q = int(rng.integers(4000, 9000))
        s = int(rng.integers(10, 21))
        bound = "fast" if rng.random() < 0.25 else "conservative"
        M, _, _ = oz.crt_constants(oz.greedy_moduli(s))
        if bound == "conservative" and oz.kbits(M, q) < 1:
            continue
        phi = float(rng.choice([0.0, 0.5, 1.0, 2.0]))
        pads = tuple(int(rng.integers(0, 4)) for _ in range(3))
        special = str(rng.choice(["none", "zero", "tiny", "huge", "nonfinite"]))
        cases.append((m, n, q, s, bound, phi, pads, special, int(rng.integers(0, 2**31))))
    return cases


ONE_PASS_CASES = draw_one_pass_cases(12)


@pytest.mark.parametrize("case", range(len(ONE_PASS_CASES)))
def test_random_one_pass_range_case(case):
    m, n, q, s, bound, phi, pads, special, seed = ONE_PASS_CASES[case]
    log(f"random one-pass-range case {case}: m={m} n={n} q={q} s={s} bound={bound} phi={phi} pads={pads} "
        f"special={special}")
    A, B = make_inputs(m, n, q, phi, special, seed)
    L.ozgemm_free()
    configure(MAX_M, MAX_N, 9000, 20)
    L.ozgemm_set_bound(L.OZGEMM_BOUND_FAST if bound == "fast" else L.OZGEMM_BOUND_CONSERVATIVE)
    try:
        C, _ = run_dgemm(A, B, s, lda=m + pads[0], ldb=q + pads[1], ldc=m + pads[2])
    finally:
        L.ozgemm_set_bound(L.OZGEMM_BOUND_CONSERVATIVE)
        L.ozgemm_free()
        configure(MAX_M, MAX_N, MAX_Q, 20)
    ref = oz.dgemm(A, B, s, bound=bound)
    assert same_doubles(C, ref), first_diff(C, ref)


# ---- 10 Scheme II cases under the OS II-accu bit budget ----

def draw_accu_cases(count: int, seed: int = 20261205):
    """The same kinds of case under OS II-accu (Ozaki II notes §9), whose
    budget depends on the range of every entry of |A'||B'|: q up to 3000,
    phi up to 16 (wide exponent ranges are what the budget is for).  Short
    and long q alternate, and the special rows and phi cycle through every
    kind and value (ten distinct pairs)."""
    kinds = ["none", "zero", "tiny", "huge", "nonfinite"]
    phis = [0.5, 1.0, 4.0, 16.0, 0.0]
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < count:
        m = int(rng.integers(1, MAX_M + 1))
        n = int(rng.integers(1, MAX_N + 1))
        q = int(rng.integers(1, 600)) if len(cases) % 2 == 0 else int(rng.integers(600, 3001))
        s = int(rng.integers(8, 21))
        M, _, _ = oz.crt_constants(oz.greedy_moduli(s))
        if oz.kbits(M, q) < 1:
            continue
        phi = phis[(len(cases) // 2) % len(phis)]
        pads = tuple(int(rng.integers(0, 4)) for _ in range(3))
        special = kinds[len(cases) % len(kinds)]
        cases.append((m, n, q, s, phi, pads, special, int(rng.integers(0, 2**31))))
    return cases


ACCU_CASES = draw_accu_cases(10)


@pytest.mark.parametrize("case", range(len(ACCU_CASES)))
def test_random_accu_case(case):
    m, n, q, s, phi, pads, special, seed = ACCU_CASES[case]
    log(f"random accu case {case}: m={m} n={n} q={q} s={s} phi={phi} pads={pads} special={special}")
    A, B = make_inputs(m, n, q, phi, special, seed)
    L.ozgemm_set_bound(L.OZGEMM_BOUND_ACCU)
    try:
        C, _ = run_dgemm(A, B, s, lda=m + pads[0], ldb=q + pads[1], ldc=m + pads[2])
    finally:
        L.ozgemm_set_bound(L.OZGEMM_BOUND_CONSERVATIVE)
    ref = oz.dgemm(A, B, s, bound="accu")
    assert same_doubles(C, ref), first_diff(C, ref)
    with np.errstate(invalid="ignore", over="ignore"):
        finite_rows = np.isfinite(A).all(axis=1)
        finite_cols = np.isfinite(B).all(axis=0)
        sub = np.ix_(finite_rows, finite_cols)
        assert within_tolerance(C[sub], ref[sub], A[finite_rows], B[:, finite_cols])


# ---- Scheme I: 16 cases of the same kinds, k in 2..10, RN or Hybrid ----

def draw_s1_cases(count: int, seed: int = 20261203):
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(count):
        m = int(rng.integers(1, MAX_M + 1))
        n = int(rng.integers(1, MAX_N + 1))
        q = int(rng.integers(1, 600)) if rng.random() < 0.5 else int(rng.integers(600, MAX_Q + 1))
        k = int(rng.integers(2, 11))
        variant = str(rng.choice(["rn", "hybrid"]))
        phi = float(rng.choice([0.0, 0.5, 1.0, 2.0, 8.0]))
        pads = tuple(int(rng.integers(0, 4)) for _ in range(3))
        special = str(rng.choice(["none", "none", "zero", "tiny", "huge", "nonfinite"]))
        cases.append((m, n, q, k, variant, phi, pads, special, int(rng.integers(0, 2**31))))
    return cases


S1_CASES = draw_s1_cases(16)


@pytest.mark.parametrize("case", range(len(S1_CASES)))
def test_random_scheme1_case(case):
    import torch
    from oracle import ozaki1 as o1
    m, n, q, k, variant, phi, pads, special, seed = S1_CASES[case]
    log(f"random Scheme I case {case}: m={m} n={n} q={q} k={k} {variant} phi={phi} pads={pads} special={special}")
    A, B = make_inputs(m, n, q, phi, special, seed)
    v = L.OZGEMM_S1_RN if variant == "rn" else L.OZGEMM_S1_HYBRID
    need = max(L.ozgemm_workspace_bytes(MAX_M, MAX_N, MAX_Q, 20), L.ozgemm_scheme1_workspace_bytes(m, n, q, k, v))
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    L.ozgemm_free()
    L.ozgemm_config(20, MAX_M, MAX_N, MAX_Q, workspace=ws)
    try:
        lda, ldb, ldc = m + pads[0], q + pads[1], m + pads[2]
        Ad = dev_colmajor(A, lda, fill=np.nan)
        Bd = dev_colmajor(B, ldb, fill=np.nan)
        Cd = torch.full((max(n, 1), ldc), 12345.0, dtype=torch.float64, device="cuda")
        L.ozgemm_scheme1_dgemm(m, n, q, Ad, lda, Bd, ldb, Cd, ldc, k, v)
        torch.cuda.synchronize()
        buf = Cd.cpu().numpy()
        C = buf[:n, :m].T
        assert np.all(buf[:n, m:] == 12345.0), "ldc padding written"
    finally:
        del ws
        configure(MAX_M, MAX_N, MAX_Q, 20)
    ref = o1.dgemm(A, B, k, variant)
    assert same_doubles(C, ref), first_diff(C, ref)
