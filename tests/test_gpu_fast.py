"""GPU parity of Scheme II under the OS II-fast bit budget (Ozaki II notes
§9): the Cauchy-Schwarz exponents e', f' and every later stage must match
the oracle's fast mode bit for bit, as in the conservative tests."""
import numpy as np
import pytest

from oracle import ozaki2 as oz
from fp64_gemm_emulation_ozii_amd import ozgemm as L
from fp64_gemm_emulation_ozii_amd.synthetic import hpl_like, integer_valued

from gpu_util import configure, first_diff, log, run_dgemm, run_stages, same_doubles
from test_gpu_parity import check_all_stages, special_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def fast_config():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    configure(1536, 1536, 1536, 20)
    L.ozgemm_set_bound(L.OZGEMM_BOUND_FAST)
    yield
    L.ozgemm_set_bound(L.OZGEMM_BOUND_CONSERVATIVE)
    L.ozgemm_free()


@pytest.mark.parametrize("s", [1, 8, 12, 13, 14, 16, 20])
def test_budget_matches_oracle(s):
    M, _, _ = oz.crt_constants(oz.greedy_moduli(s))
    assert L.ozgemm_bound_budget(s, 1000, L.OZGEMM_BOUND_FAST) == oz.cs_budget(M)


def test_tiny_64_cube_s14_all_stages():
    A, B = hpl_like(64, 64, 64, 0.5, seed=0)
    log("fast tiny 64^3 s=14")
    check_all_stages(A, B, 14, run_stages(A, B, 14), bound="fast")


@pytest.mark.parametrize("shape", [(1, 1, 1), (7, 13, 5), (65, 127, 129), (300, 257, 1000), (257, 255, 129)])
@pytest.mark.parametrize("s", [8, 12, 13, 14])
def test_ragged_shapes(shape, s):
    m, q, n = shape
    A, B = hpl_like(m, q, n, 1.0, seed=m + q + n)
    log(f"fast ragged m={m} q={q} n={n} s={s}")
    check_all_stages(A, B, s, run_stages(A, B, s), bound="fast")


@pytest.mark.parametrize("s", [10, 14, 18])
def test_special_values(s):
    A, B = special_inputs()
    log(f"fast special values s={s}")
    check_all_stages(A, B, s, run_stages(A, B, s), bound="fast")


def test_integer_inputs_exact():
    A, B = integer_valued(100, 64, 90, 2**10, seed=2)
    C, _ = run_dgemm(A, B, 14)
    assert np.array_equal(C, A @ B)


def test_1024_cube_full_oracle():
    A, B = hpl_like(1024, 1024, 1024, 0.5, seed=0)
    log("fast 1024^3 s=14: GPU")
    g = run_stages(A, B, 14, want_ct=False, want_prime=True)
    log("fast 1024^3 s=14: oracle")
    ref = oz.dgemm(A, B, 14, stages=True, bound="fast")
    check_all_stages(A, B, 14, g, ref=ref, bound="fast")


def test_more_correct_bits_than_conservative():
    A, B = hpl_like(256, 512, 256, 1.0, seed=9)
    rng = np.random.default_rng(3)
    rows, cols = rng.integers(0, 256, 40), rng.integers(0, 256, 40)
    Cf, _ = run_dgemm(A, B, 12)
    L.ozgemm_set_bound(L.OZGEMM_BOUND_CONSERVATIVE)
    try:
        Cc, _ = run_dgemm(A, B, 12)
    finally:
        L.ozgemm_set_bound(L.OZGEMM_BOUND_FAST)
    bf = oz.correct_bits(Cf, A, B, rows, cols)
    bc = oz.correct_bits(Cc, A, B, rows, cols)
    log(f"fast {bf:.2f} bits vs conservative {bc:.2f}")
    assert bf >= bc + 2.0


def test_sampled_8192_cube():
    import torch
    m = n = q = 8192
    s = 14
    A, B = hpl_like(m, q, n, 1.0, seed=0)
    L.ozgemm_free()
    L.ozgemm_config(s, m, n, q)
    L.ozgemm_set_bound(L.OZGEMM_BOUND_FAST)
    try:
        Ad = torch.from_numpy(np.ascontiguousarray(A.T)).cuda()
        Bd = torch.from_numpy(np.ascontiguousarray(B.T)).cuda()
        Cd = torch.empty((n, m), dtype=torch.float64, device="cuda")
        e = torch.empty(m, dtype=torch.int32, device="cuda")
        f = torch.empty(n, dtype=torch.int32, device="cuda")
        log("fast 8192^3: GPU")
        L.ozgemm_dgemm(m, n, q, Ad, m, Bd, q, Cd, m, s)
        L.ozgemm_stage_scale(m, n, q, s, Ad, m, Bd, q, e, f)
        torch.cuda.synchronize()
        rng = np.random.default_rng(12345)
        rows = np.unique(np.concatenate([rng.integers(0, m, 48), [0, m - 1]]))
        cols = np.unique(np.concatenate([rng.integers(0, n, 48), [0, n - 1]]))
        Cg = Cd.T[torch.from_numpy(rows).cuda()][:, torch.from_numpy(cols).cuda()].cpu().numpy()
        eg, fg = e.cpu().numpy(), f.cpu().numpy()
        del Ad, Bd, Cd
        torch.cuda.empty_cache()
    finally:
        L.ozgemm_free()
        configure(1536, 1536, 1536, 20)
        L.ozgemm_set_bound(L.OZGEMM_BOUND_FAST)
    log("fast 8192^3: oracle exponents")
    M, _, _ = oz.crt_constants(oz.greedy_moduli(s))
    kA, kB = oz.cs_budget(M)
    kb = max(kA, kB)
    assert np.array_equal(eg, oz.fast_exponents(A, oz.row_exponents(A), kA, kb)), "row exponents"
    assert np.array_equal(fg, oz.fast_exponents(B.T, oz.col_exponents(B), kB, kb)), "column exponents"
    log("fast 8192^3: oracle block")
    ref = oz.dgemm_block(A, B, s, rows, cols, bound="fast")
    assert same_doubles(Cg, ref), first_diff(Cg, ref)
