"""GPU parity: every stage of the HIP path against the oracle.

Integer stages (exponents, A', B', int8 residue planes, int32 products,
product residues) must match bit for bit; the FP64 result must lie within
2^-50 (|A||B|)_ij of the oracle's correctly rounded value (the required
tolerance) and, because the CRT kernel also rounds once to nearest, is
expected to match it bit for bit as well.
"""
import numpy as np
import pytest

from oracle import ozaki2 as oz
from fp64_gemm_emulation_ozii_amd import ozgemm as L
from fp64_gemm_emulation_ozii_amd.synthetic import hpl_like, integer_valued

from gpu_util import configure, first_diff, log, run_dgemm, run_stages, same_doubles, within_tolerance

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def small_config():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    configure(1536, 1536, 1536, 20)
    yield
    L.ozgemm_free()


def check_all_stages(A, B, s, g, ref=None, bound="conservative"):
    """Compare every stage of run_stages output g with the oracle."""
    C_ref, st = ref if ref is not None else oz.dgemm(A, B, s, stages=True, bound=bound)
    m, q = A.shape
    n = B.shape[1]
    assert np.array_equal(g["e"], st["e"]), first_diff(g["e"], st["e"])
    assert np.array_equal(g["f"], st["f"]), first_diff(g["f"], st["f"])
    if "Ap" in g:
        assert np.array_equal(g["Ap"], st["Ap"]), first_diff(g["Ap"], st["Ap"])
        assert np.array_equal(g["Bp"], st["Bp"]), first_diff(g["Bp"], st["Bp"])
    assert np.array_equal(g["Ares"], st["Ares"]), first_diff(g["Ares"], st["Ares"])
    assert np.array_equal(g["Bres"], st["Bres"]), first_diff(g["Bres"], st["Bres"])
    # the padding of the planes is zero
    assert not g["Ares_full"][:, m:, :].any() and not g["Ares_full"][:, :, q:].any()
    assert not g["Bres_full"][:, n:, :].any() and not g["Bres_full"][:, :, q:].any()
    if "Ct" in g:
        assert np.array_equal(g["Ct"], st["Ct"]), first_diff(g["Ct"], st["Ct"])
    assert np.array_equal(g["rt"], st["rt"]), first_diff(g["rt"], st["rt"])
    assert within_tolerance(g["C"], C_ref, A, B)
    assert same_doubles(g["C"], C_ref), first_diff(g["C"], C_ref)


def test_tiny_64_cube_s14_all_stages():
    """64 x 64 x 64, HPL-like phi = 0.5, seed 0, s = 14."""
    A, B = hpl_like(64, 64, 64, 0.5, seed=0)
    log("tiny 64^3 s=14")
    check_all_stages(A, B, 14, run_stages(A, B, 14))


@pytest.mark.parametrize("shape", [(1, 1, 1), (7, 13, 5), (65, 127, 129), (129, 65, 1280), (300, 257, 1000),
                                   (33, 500, 2), (256, 256, 128), (257, 255, 129)])
@pytest.mark.parametrize("s", [8, 14])
def test_ragged_shapes(shape, s):
    m, q, n = shape
    M, _, _ = oz.crt_constants(oz.greedy_moduli(s))
    if oz.kbits(M, q) < 1:
        pytest.skip("no bits left")
    A, B = hpl_like(m, q, n, 1.0, seed=m + q + n)
    log(f"ragged m={m} q={q} n={n} s={s}")
    # without int32 planes the GEMM takes its residue-only epilogue (staged
    # through LDS); with them, the direct one
    check_all_stages(A, B, s, run_stages(A, B, s, want_ct=(s == 14)))


@pytest.mark.parametrize("s,q", [(16, 64), (18, 64), (18, 1000), (20, 3), (20, 200)])
def test_k_above_53(s, q):
    """k > 53: A' no longer fits the 53-bit significand (residues via u 2^sh)."""
    M, _, _ = oz.crt_constants(oz.greedy_moduli(s))
    assert oz.kbits(M, q) > 53
    A, B = hpl_like(40, q, 33, 0.5, seed=s)
    log(f"k>53 s={s} q={q}")
    check_all_stages(A, B, s, run_stages(A, B, s))


def special_inputs():
    rng = np.random.default_rng(21)
    A, B = hpl_like(70, 90, 66, 2.0, seed=5)
    A[0, :] = 0.0                          # zero row -> +0
    B[:, 1] = 0.0                          # zero column
    A[2, 17] = np.inf                      # non-finite row -> NaN row
    B[30, 3] = np.nan                      # non-finite column
    A[4, :] = rng.standard_normal(90) * 1e-310   # subnormal-ish row
    A[5, :] = rng.standard_normal(90) * 1e300    # near-overflow row
    B[:, 6] = rng.standard_normal(90) * 1e300    # overflow products -> +-Inf
    A[7, :] = rng.standard_normal(90) * 1e-300
    B[:, 8] = rng.standard_normal(90) * 1e-300   # underflow products -> subnormal / 0
    A[9, :] = 2.0 ** 40                    # exact powers of two
    A[10, 3] = -5e-324                     # lone smallest subnormal in a normal row
    return A, B


@pytest.mark.parametrize("s", [10, 14, 18])
def test_special_values(s):
    A, B = special_inputs()
    log(f"special values s={s}")
    check_all_stages(A, B, s, run_stages(A, B, s))


def test_integer_inputs_exact():
    A, B = integer_valued(100, 64, 90, 2**10, seed=2)
    C, _ = run_dgemm(A, B, 14)
    assert np.array_equal(C, A @ B)


def test_leading_dimension_padding():
    A, B = hpl_like(45, 77, 31, 1.0, seed=3)
    C0, _ = run_dgemm(A, B, 14)
    C1, buf = run_dgemm(A, B, 14, lda=50, ldb=80, ldc=47)
    assert same_doubles(C0, C1)
    # entries of C's padding rows are untouched
    assert np.all(buf[:31, 45:47] == 12345.0)
    g = run_stages(A, B, 14, lda=64, ldb=128, ldc=64)
    assert same_doubles(g["C"], C0)


def test_dgemm_matches_stages_and_oracle():
    A, B = hpl_like(200, 333, 150, 0.5, seed=4)
    C, _ = run_dgemm(A, B, 14)
    g = run_stages(A, B, 14, want_ct=False, want_prime=False)
    assert same_doubles(C, g["C"])
    assert same_doubles(C, oz.dgemm(A, B, 14))


def test_q_zero_writes_zero_and_empty_shapes():
    import torch
    Cd = torch.full((5, 4), 3.0, dtype=torch.float64, device="cuda")
    dummy = torch.zeros(8, dtype=torch.float64, device="cuda")
    L.ozgemm_dgemm(4, 5, 0, dummy, 4, dummy, 1, Cd, 4, 14)
    torch.cuda.synchronize()
    assert torch.all(Cd == 0).item()
    L.ozgemm_dgemm(0, 5, 3, dummy, 1, dummy, 3, Cd, 1, 14)
    L.ozgemm_dgemm(4, 0, 3, dummy, 4, dummy, 3, Cd, 4, 14)


@pytest.mark.parametrize("bound", ["conservative", "fast"])
def test_stage_scale_empty_inner_dimension(bound):
    """q = 0 through the scale entry point: every row and column is empty,
    so each exponent is the oracle's exponent of an empty row (0) under both
    budgets; no entry of A or B is read."""
    import torch
    m, n = 300, 200
    A, B = np.zeros((m, 0)), np.zeros((0, n))
    want_e = oz.row_exponents(A)
    want_f = oz.col_exponents(B)
    if bound == "fast":
        ka, kb = oz.cs_budget(oz.crt_constants(oz.greedy_moduli(14))[0])
        base = max(ka, kb)
        want_e = oz.fast_exponents(A, want_e, ka, base)
        want_f = oz.fast_exponents(B.T, want_f, kb, base)
    dummy = torch.zeros(8, dtype=torch.float64, device="cuda")
    e = torch.full((m,), -7, dtype=torch.int32, device="cuda")
    f = torch.full((n,), -7, dtype=torch.int32, device="cuda")
    log(f"stage_scale q = 0, {bound}")
    L.ozgemm_set_bound(L.OZGEMM_BOUND_FAST if bound == "fast" else L.OZGEMM_BOUND_CONSERVATIVE)
    try:
        L.ozgemm_stage_scale(m, n, 0, 14, dummy, m, dummy, 1, e, f)
        torch.cuda.synchronize()
    finally:
        L.ozgemm_set_bound(L.OZGEMM_BOUND_CONSERVATIVE)
    assert np.array_equal(e.cpu().numpy(), want_e)
    assert np.array_equal(f.cpu().numpy(), want_f)


def test_invariants_on_gpu():
    A, B = hpl_like(60, 70, 50, 1.0, seed=8)
    C, _ = run_dgemm(A, B, 14)
    C2, _ = run_dgemm(A * 2.0**-30, B, 14)
    assert same_doubles(C2, C * 2.0**-30)
    Cn, _ = run_dgemm(-A, B, 14)
    assert same_doubles(Cn, -C)
    Ct, _ = run_dgemm(B.T.copy(), A.T.copy(), 14)
    assert same_doubles(Ct, C.T)


def test_phase_timing():
    import torch
    A, B = hpl_like(128, 128, 128, 0.5, seed=1)
    L.ozgemm_timing(True)
    for _ in range(3):
        run_dgemm(A, B, 14)
    ms, calls = L.ozgemm_phase_ms()
    L.ozgemm_timing(False)
    assert calls == 3 and all(x > 0 for x in ms)


@pytest.mark.parametrize("s", [8, 14, 18])
def test_1024_cube_full_oracle(s):
    """1024^3, phi = 0.5: integer stages (s = 14) and the full result bit-exact."""
    A, B = hpl_like(1024, 1024, 1024, 0.5, seed=0)
    log(f"1024^3 s={s}: GPU")
    g = run_stages(A, B, s, want_ct=(s == 14), want_prime=(s == 14))
    log(f"1024^3 s={s}: oracle")
    ref = oz.dgemm(A, B, s, stages=True)
    log(f"1024^3 s={s}: compare")
    check_all_stages(A, B, s, g, ref=ref)


@pytest.mark.parametrize("s,q", [(14, 2**17 + 300), (10, 140000), (14, 2**17 - 100)])
def test_long_inner_dimension(s, q):
    """q >= 2^17: the GEMM cuts K into parts of at most 2^16 (block
    products), here run as K parts of one launch; residues of the products
    and C must still match."""
    import torch
    A, B = hpl_like(65, q, 70, 1.0, seed=q % 1000)
    L.ozgemm_free()
    configure(256, 256, q, 20)
    try:
        assert L.ozgemm_gemm_parts(65, 70, q, s) >= 2
        log(f"long K s={s} q={q}")
        g = run_stages(A, B, s, want_ct=q < 2**17, want_prime=True)
        C, _ = run_dgemm(A, B, s)
    finally:
        L.ozgemm_free()
        torch.cuda.empty_cache()
        configure(1536, 1536, 1536, 20)
    ref = oz.dgemm(A, B, s, stages=True)
    check_all_stages(A, B, s, g, ref=ref)
    assert same_doubles(C, ref[0])


@pytest.mark.parametrize("m,q,n,s,parts", [(300, 5000, 200, 14, 2), (65, 9000, 70, 8, 4), (257, 4200, 513, 13, 2)])
def test_k_parts(m, q, n, s, parts):
    """Skinny outputs with a long inner dimension run as K parts: one block
    per (part, modulus, tile), each part's product mod m_t in a plane of its
    own, then the parts summed mod m_t.  With 8 | parts * s a plane's tiles
    also sit on one XCD.  Every stage must still match the oracle."""
    import torch
    A, B = hpl_like(m, q, n, 1.0, seed=m + q + n)
    L.ozgemm_free()
    configure(1536, 1536, 9000, 20)
    try:
        assert L.ozgemm_gemm_parts(m, n, q, s) == parts
        log(f"K parts m={m} q={q} n={n} s={s} parts={parts}")
        g = run_stages(A, B, s, want_ct=False)  # int32 planes would keep one part
        C, _ = run_dgemm(A, B, s)
    finally:
        L.ozgemm_free()
        torch.cuda.empty_cache()
        configure(1536, 1536, 1536, 20)
    ref = oz.dgemm(A, B, s, stages=True)
    check_all_stages(A, B, s, g, ref=ref)
    assert same_doubles(C, ref[0])


@pytest.mark.parametrize("m,q,n,s", [(700, 512, 900, 14), (1100, 129, 520, 11), (257, 384, 1536, 16)])
def test_short_inner_dimension(m, q, n, s):
    """K <= 512 (at most four K slices per block): residue-only products run
    eight wavefronts per block; several row and column tiles, ragged."""
    A, B = hpl_like(m, q, n, 1.0, seed=m * 7 + q)
    log(f"short K m={m} q={q} n={n} s={s}")
    ref = oz.dgemm(A, B, s, stages=True)
    check_all_stages(A, B, s, run_stages(A, B, s, want_ct=False), ref=ref)
    C, _ = run_dgemm(A, B, s)
    assert same_doubles(C, ref[0])


@pytest.mark.parametrize("m,n,q,parts", [(1100, 1000, 2048, 1), (1100, 1000, 2049, 1), (300, 520, 2048, 1),
                                         (300, 520, 2049, 1), (256, 200, 4096, 2), (256, 200, 4224, 2)])
def test_eight_wave_boundary(m, n, q, parts):
    """Residue-only products whose blocks walk at most 16 K slices of 128
    run eight wavefronts per block, longer ones four: q = 2048 and 2049 on
    either side, each in the persistent grid (20 tiles x 14 moduli > 256
    compute units) and with one block per tile (6 x 14); and a single tile
    cut into two K parts of 16 slices (q = 4096) and of 17 (q = 4224).
    Every stage must match the oracle."""
    import torch
    A, B = hpl_like(m, q, n, 1.0, seed=m + n + q)
    L.ozgemm_free()
    configure(1536, 1536, 4224, 20)
    try:
        assert L.ozgemm_gemm_parts(m, n, q, 14) == parts
        log(f"eight-wave boundary m={m} n={n} q={q}")
        g = run_stages(A, B, 14, want_ct=False)  # int32 planes would take the four-wavefront debug form
        C, _ = run_dgemm(A, B, 14)
    finally:
        L.ozgemm_free()
        torch.cuda.empty_cache()
        configure(1536, 1536, 1536, 20)
    ref = oz.dgemm(A, B, 14, stages=True)
    check_all_stages(A, B, 14, g, ref=ref)
    assert same_doubles(C, ref[0])


def test_long_inner_dimension_refuses_int32_planes():
    import torch
    L.ozgemm_free()
    configure(256, 256, 2**17 + 128, 14)
    try:
        z8 = torch.zeros(14 * 256 * (2**17 + 128), dtype=torch.int8, device="cuda")
        ct = torch.zeros(14 * 256 * 256, dtype=torch.int32, device="cuda")
        st = L.ozgemm_stage_gemm(10, 10, 2**17 + 1, 14, z8, z8, ct, None, check=False)
        assert st == L.OZGEMM_RANGE
    finally:
        L.ozgemm_free()
        configure(1536, 1536, 1536, 20)


@pytest.mark.parametrize("q", [L.OZGEMM_ONE_PASS_Q_MIN - 1, L.OZGEMM_ONE_PASS_Q_MIN, L.OZGEMM_ONE_PASS_Q_MIN + 37,
                               L.OZGEMM_ONE_PASS_Q_MAX, L.OZGEMM_ONE_PASS_Q_MAX + 1])
@pytest.mark.parametrize("bound", ["conservative", "fast"])
def test_b_one_pass_boundary(q, bound):
    """For OZGEMM_ONE_PASS_Q_MIN <= q <= OZGEMM_ONE_PASS_Q_MAX ozgemm_dgemm
    takes B's column exponents (under OS II-fast with the columns' norm
    bounds) inside its residue pass (B read once); outside that range the
    scale step does.
    Columns of B that are all zero, subnormal only, near overflow or hold a
    NaN exercise that exponent; C must equal the oracle bit for bit either
    way, and the stage entry points (always two passes) must agree."""
    import torch
    m, n = 70, 300
    A, B = hpl_like(m, q, n, 1.0, seed=q)
    B[:, 3] = 0.0
    B[:, 5] *= 2.0 ** -1060          # every entry subnormal
    B[:, 7] *= 2.0 ** 1000
    B[q // 2, 11] = np.nan
    B[q - 1, 13] = 2.0 ** -1074      # the column maximum sits in the last entry
    B[:q - 1, 13] = 2.0 ** -1075 * 0.0
    L.ozgemm_free()
    configure(256, 512, q, 20)
    L.ozgemm_set_bound(L.OZGEMM_BOUND_FAST if bound == "fast" else L.OZGEMM_BOUND_CONSERVATIVE)
    try:
        log(f"one-pass boundary q={q} bound={bound}")
        C, _ = run_dgemm(A, B, 14)
        g = run_stages(A, B, 14, want_ct=False, want_prime=False)
    finally:
        L.ozgemm_set_bound(L.OZGEMM_BOUND_CONSERVATIVE)
        L.ozgemm_free()
        torch.cuda.empty_cache()
        configure(1536, 1536, 1536, 20)
    ref = oz.dgemm(A, B, 14, stages=True, bound=bound)
    assert same_doubles(C, ref[0]), first_diff(C, ref[0])
    assert np.array_equal(g["f"], ref[1]["f"]), first_diff(g["f"], ref[1]["f"])
    assert same_doubles(g["C"], C)
