"""GPU parity of the Scheme I path (slice split, slice products, FP64
accumulation) against the oracle in oracle/ozaki1.py.

Slices, grid exponents and int32 products must match bit for bit.  The FP64
accumulation adds exact terms in the same fixed order on both sides, so C
must match bit for bit too (and lies within 2^-50 (|A||B|)_ij of it
trivially).  Large problems are checked on a block of rows and columns: the
split of a row (column) depends on that row (column) alone, so the oracle
run on the selected rows of A and columns of B gives exactly those entries.
"""
import numpy as np
import pytest

from oracle import ozaki1 as o1
from fp64_gemm_emulation_ozii_amd import ozgemm as L
from fp64_gemm_emulation_ozii_amd.synthetic import hpl_like

from gpu_util import dev_colmajor, first_diff, log, same_doubles

pytestmark = pytest.mark.gpu

VARIANTS = {"rn": L.OZGEMM_S1_RN, "hybrid": L.OZGEMM_S1_HYBRID}
NONF = L.OZGEMM_EXP_NONFINITE


def reconfigure(m, n, q, k, variant):
    """Configure with a workspace large enough for Scheme I at (m, n, q, k)."""
    import torch
    L.ozgemm_free()
    need = max(L.ozgemm_workspace_bytes(256, 256, 256, 14), L.ozgemm_scheme1_workspace_bytes(m, n, q, k, variant))
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    L.ozgemm_config(14, 256, 256, 256, workspace=ws)


@pytest.fixture(scope="module", autouse=True)
def config():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    # workspace sized for the largest stage-level case below
    reconfigure(1024, 1024, 1024, 8, L.OZGEMM_S1_RN)
    yield
    L.ozgemm_free()


def run_s1_stages(A, B, k, variant):
    import torch
    m, q = A.shape
    n = B.shape[1]
    v = VARIANTS[variant]
    Ad = dev_colmajor(A, max(1, m), fill=np.nan)
    Bd = dev_colmajor(B, max(1, q), fill=np.nan)
    mp, np_, qp = L.ozgemm_plane_dims(m, n, q)
    rows = k if variant == "rn" else 1
    nout = L.ozgemm_scheme1_outputs(k, v, q)
    dev = "cuda"
    Asl = torch.full((k * mp * qp,), 99, dtype=torch.int8, device=dev)
    Bsl = torch.full((k * np_ * qp,), 99, dtype=torch.int8, device=dev)
    gA = torch.full((rows * mp,), -7, dtype=torch.int32, device=dev)
    gB = torch.full((rows * np_,), -7, dtype=torch.int32, device=dev)
    P = torch.full((nout * mp * np_,), 7, dtype=torch.int32, device=dev)
    Cd = torch.full((max(n, 1), max(m, 1)), 12345.0, dtype=torch.float64, device=dev)
    L.ozgemm_scheme1_stage_split(m, n, q, k, v, Ad, max(1, m), Bd, max(1, q), Asl, Bsl, gA, gB)
    L.ozgemm_scheme1_stage_products(m, n, q, k, v, Asl, Bsl, P)
    L.ozgemm_scheme1_stage_accumulate(m, n, q, k, v, P, gA, gB, Cd, max(1, m))
    torch.cuda.synchronize()
    Cf = torch.full((max(n, 1), max(m, 1)), 12345.0, dtype=torch.float64, device=dev)
    L.ozgemm_scheme1_dgemm(m, n, q, Ad, max(1, m), Bd, max(1, q), Cf, max(1, m), k, v)
    torch.cuda.synchronize()
    Asl_f = Asl.cpu().numpy().reshape(k, mp, qp)
    Bsl_f = Bsl.cpu().numpy().reshape(k, np_, qp)
    return {
        "As": Asl_f[:, :m, :q], "As_full": Asl_f,
        "Bs": Bsl_f[:, :n, :q].transpose(0, 2, 1), "Bs_full": Bsl_f,
        "gA": gA.cpu().numpy().reshape(rows, mp)[:, :m],
        "gB": gB.cpu().numpy().reshape(rows, np_)[:, :n],
        "P": P.cpu().numpy().reshape(nout, np_, mp)[:, :n, :m].transpose(0, 2, 1),
        "C": Cd.cpu().numpy()[:n, :m].T,
        "C_dgemm": Cf.cpu().numpy()[:n, :m].T,
    }


def expected_grids(X, g, variant):
    """Oracle grid exponents in the library's layout (one row for Hybrid;
    the first row carries the non-finite flag)."""
    g = np.array(g, dtype=np.int64).reshape(-1, X.shape[0]) if variant == "rn" else np.array(g).reshape(1, -1)
    bad = ~np.all(np.isfinite(X), axis=1)
    g = g.copy()
    g[0, bad] = NONF
    return g


def check_parity(A, B, k, variant):
    m, q = A.shape
    n = B.shape[1]
    C_ref, st = o1.dgemm(A, B, k, variant, stages=True)
    gpu = run_s1_stages(A, B, k, variant)
    assert np.array_equal(gpu["As"], st["As"]), first_diff(gpu["As"], st["As"])
    assert np.array_equal(gpu["Bs"], st["Bs"]), first_diff(gpu["Bs"], st["Bs"])
    assert not gpu["As_full"][:, m:, :].any() and not gpu["As_full"][:, :, q:].any()
    assert not gpu["Bs_full"][:, n:, :].any() and not gpu["Bs_full"][:, :, q:].any()
    eA = expected_grids(A, st["gA"], variant)
    eB = expected_grids(B.T, st["gB"], variant)
    assert np.array_equal(gpu["gA"], eA), first_diff(gpu["gA"], eA)
    assert np.array_equal(gpu["gB"], eB), first_diff(gpu["gB"], eB)
    ref_P = np.stack(st["products"])
    assert np.array_equal(gpu["P"], ref_P), first_diff(gpu["P"], ref_P)
    assert same_doubles(gpu["C"], C_ref), first_diff(gpu["C"], C_ref)
    assert same_doubles(gpu["C_dgemm"], C_ref), first_diff(gpu["C_dgemm"], C_ref)


@pytest.mark.parametrize("variant", ["rn", "hybrid"])
@pytest.mark.parametrize("shape,k", [((1, 1, 1), 4), ((7, 13, 5), 8), ((65, 127, 129), 8), ((129, 65, 300), 6),
                                     ((300, 257, 1000), 4), ((257, 255, 129), 8), ((64, 64, 64), 1)])
def test_parity_ragged(variant, shape, k):
    m, n, q = shape
    A, B = hpl_like(m, q, n, 1.0, seed=m + n + q)
    log(f"scheme1 {variant} k={k} {shape}")
    check_parity(A, B, k, variant)


@pytest.mark.parametrize("variant", ["rn", "hybrid"])
def test_special_values(variant):
    rng = np.random.default_rng(17)
    m, n, q = 70, 40, 150
    A = (rng.random((m, q)) - 0.5) * np.exp(2 * rng.standard_normal((m, q)))
    B = (rng.random((q, n)) - 0.5) * np.exp(2 * rng.standard_normal((q, n)))
    A[0, :] = 0.0
    A[1, 7] = np.inf
    A[2, 9] = np.nan
    A[3, :] *= 2.0**1000        # huge row
    A[4, :] *= 2.0**-1060       # subnormal row
    A[5, :] = 2.0**-1074        # smallest subnormal
    A[6, ::2] = 0.0
    A[7, :] = 1.0               # exact power of two maximum
    B[:, 0] = 0.0
    B[5, 1] = -np.inf
    B[:, 2] *= 2.0**-1000
    B[:, 3] = -4.0
    log(f"scheme1 special {variant}")
    check_parity(A, B, 6, variant)


@pytest.mark.parametrize("variant", ["rn", "hybrid"])
@pytest.mark.parametrize("q", [150, L.OZGEMM_ONE_PASS_Q_MIN])
def test_rows_near_the_largest_double(variant, q):
    """Rows of A and columns of B whose maximum is within one grid step of the
    largest double: the first slice's grid times 2^(beta-1) is 2^1024, and the
    residual must still be the exact difference.  B's columns are split by the
    multi-pass kernels at q = 150 and by the one-pass kernel at q = 4096."""
    rng = np.random.default_rng(23)
    m, n = 40, 24
    big = np.nextafter(np.inf, 0.0)
    A = (rng.random((m, q)) - 0.5) * np.exp(rng.standard_normal((m, q)))
    B = (rng.random((q, n)) - 0.5) * np.exp(rng.standard_normal((q, n))) * 2.0**-1000
    A[0, 3], A[0, 5] = big, -0.75 * big
    A[1, 0] = 1.9921875 * 2.0**1023
    A[2, :] = np.ldexp(A[2, :] / np.abs(A[2, :]).max(), 1023)
    A[2, 1] = -big
    Bb = (rng.random((q, n)) - 0.5) * 2.0**-40
    Bb[4, 0], Bb[7, 1] = big, -big
    B[:, :2] = Bb[:, :2]  # two columns of B near the top too (against finite rows of A only)
    A2 = A * 2.0**-30
    A2[:3, :] = 0.0
    log(f"scheme1 near-overflow {variant} q={q}")
    check_parity(A, B[:, 2:], 6, variant)
    check_parity(A2, B, 6, variant)


@pytest.mark.parametrize("variant", ["rn", "hybrid"])
def test_small_integers_exact(variant):
    rng = np.random.default_rng(2)
    A = rng.integers(-63, 64, size=(100, 333)).astype(np.float64)
    B = rng.integers(-63, 64, size=(333, 77)).astype(np.float64)
    A[:, 0] = 63.0
    B[0, :] = 63.0
    gpu = run_s1_stages(A, B, 3, variant)
    exact = (A.astype(np.int64) @ B.astype(np.int64)).astype(np.float64)
    assert np.array_equal(gpu["C"], exact)


@pytest.mark.parametrize("variant", ["rn", "hybrid"])
def test_inner_dimension_beyond_int8_scheme2_limit(variant):
    """q > 2^17: beta drops to 6 and Hybrid sums runs of r = 2 products."""
    m, n, q = 24, 20, 140000
    assert L.ozgemm_scheme1_beta(q) == 6
    A, B = hpl_like(m, q, n, 0.5, seed=4)
    reconfigure(m, n, q, 4, VARIANTS[variant])
    log(f"scheme1 {variant} q={q}")
    check_parity(A, B, 4, variant)
    reconfigure(1024, 1024, 1024, 8, L.OZGEMM_S1_RN)


@pytest.mark.parametrize("variant", ["rn", "hybrid"])
@pytest.mark.parametrize("q", [L.OZGEMM_ONE_PASS_Q_MIN - 1, L.OZGEMM_ONE_PASS_Q_MIN, L.OZGEMM_ONE_PASS_Q_MIN + 37,
                               L.OZGEMM_ONE_PASS_Q_MAX, L.OZGEMM_ONE_PASS_Q_MAX + 1])
def test_row_split_one_pass_boundary(variant, q):
    """For OZGEMM_ONE_PASS_Q_MIN <= q <= OZGEMM_ONE_PASS_Q_MAX the rows of B
    (columns, contiguous in memory) are split in one pass from LDS; outside
    that range by the rowmax, grid and split passes.  Columns of B that are
    zero, subnormal only, near overflow, hold a NaN, or whose residual
    vanishes after one slice check grids, slices, products and C bit for
    bit against the oracle either way."""
    m, n, k = 24, 40, 6
    A, B = hpl_like(m, q, n, 1.0, seed=q + 17)
    B[:, 2] = 0.0
    B[:, 4] *= 2.0 ** -1060
    B[:, 6] *= 2.0 ** 1000
    B[q // 3, 8] = np.nan
    B[:, 10] = 0.0
    B[::7, 10] = 3.0                 # exact in one slice: the residual is zero after it
    reconfigure(m, n, q, k, VARIANTS[variant])
    log(f"scheme1 {variant} one-pass boundary q={q}")
    check_parity(A, B, k, variant)
    reconfigure(1024, 1024, 1024, 8, L.OZGEMM_S1_RN)


@pytest.mark.parametrize("variant", ["rn", "hybrid"])
@pytest.mark.parametrize("size,k", [(1024, 8), (4096, 8), (4096, 5)])
def test_large_sampled_block(variant, size, k):
    import torch
    m = n = q = size
    A, B = hpl_like(m, q, n, 1.0, seed=0)
    v = VARIANTS[variant]
    reconfigure(m, n, q, k, v)
    rng = np.random.default_rng(12345)
    rows = np.unique(np.concatenate([rng.integers(0, m, 40), [0, m - 1]]))
    cols = np.unique(np.concatenate([rng.integers(0, n, 40), [0, n - 1]]))
    log(f"scheme1 {variant} {size}^3 k={k}")
    Ad = torch.from_numpy(np.ascontiguousarray(A.T)).cuda()
    Bd = torch.from_numpy(np.ascontiguousarray(B.T)).cuda()
    Cd = torch.empty((n, m), dtype=torch.float64, device="cuda")
    L.ozgemm_scheme1_dgemm(m, n, q, Ad, m, Bd, q, Cd, m, k, v)
    torch.cuda.synchronize()
    C = Cd.T[torch.from_numpy(rows).cuda()][:, torch.from_numpy(cols).cuda()].cpu().numpy()
    ref = o1.dgemm(A[rows, :], B[:, cols], k, variant)
    assert same_doubles(C, ref), first_diff(C, ref)
    del Ad, Bd, Cd
    torch.cuda.empty_cache()
    reconfigure(1024, 1024, 1024, 8, L.OZGEMM_S1_RN)


def test_workspace_too_small_is_reported():
    import torch
    L.ozgemm_free()
    L.ozgemm_config(14, 256, 256, 256)  # Scheme II sized
    m = n = q = 1024
    A = torch.zeros((q, m), dtype=torch.float64, device="cuda")
    B = torch.zeros((n, q), dtype=torch.float64, device="cuda")
    C = torch.zeros((n, m), dtype=torch.float64, device="cuda")
    st = L.ozgemm_scheme1_dgemm(m, n, q, A, m, B, q, C, m, 8, L.OZGEMM_S1_RN, check=False)
    assert st == L.OZGEMM_WORKSPACE_TOO_SMALL
    reconfigure(1024, 1024, 1024, 8, L.OZGEMM_S1_RN)
