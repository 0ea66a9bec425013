"""GPU parity of Scheme II under the OS II-accu bit budget (Ozaki II notes
§9): the band bound, the row and column bit counts and every later stage
are exact integer functions of the inputs, so the exponents e', f', the
truncated matrices, residues, products and C must match the oracle's accu
mode bit for bit."""
import numpy as np
import pytest

from oracle import ozaki2 as oz
from fp64_gemm_emulation_ozii_amd import ozgemm as L
from fp64_gemm_emulation_ozii_amd.synthetic import hpl_like, integer_valued

from gpu_util import configure, dev_colmajor, first_diff, log, run_dgemm, run_stages, same_doubles
from test_gpu_parity import check_all_stages, special_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def accu_config():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    configure(1536, 1536, 4224, 20)
    L.ozgemm_set_bound(L.OZGEMM_BOUND_ACCU)
    yield
    L.ozgemm_set_bound(L.OZGEMM_BOUND_CONSERVATIVE)
    L.ozgemm_free()


@pytest.mark.parametrize("s", [2, 8, 14, 20])
def test_budget(s):
    M, _, _ = oz.crt_constants(oz.greedy_moduli(s))
    if oz.kbits(M, 1000) < 1:
        with pytest.raises(L.OzgemmError):
            L.ozgemm_bound_budget(s, 1000, L.OZGEMM_BOUND_ACCU)
        return
    K2 = (M // 2 - 1).bit_length() - 1
    assert L.ozgemm_bound_budget(s, 1000, L.OZGEMM_BOUND_ACCU) == (K2, oz.ACCU_KMAX)


def test_tiny_64_cube_s14_all_stages():
    A, B = hpl_like(64, 64, 64, 0.5, seed=0)
    log("accu tiny 64^3 s=14")
    check_all_stages(A, B, 14, run_stages(A, B, 14), bound="accu")


@pytest.mark.parametrize("shape", [(1, 1, 1), (7, 13, 5), (65, 127, 129), (300, 257, 1000), (257, 255, 129),
                                   (129, 4097, 65)])
@pytest.mark.parametrize("s", [8, 14])
@pytest.mark.parametrize("phi", [0.5, 4.0])
def test_ragged_shapes(shape, s, phi):
    m, q, n = shape
    A, B = hpl_like(m, q, n, phi, seed=m + q + n)
    log(f"accu ragged m={m} q={q} n={n} s={s} phi={phi}")
    check_all_stages(A, B, s, run_stages(A, B, s, want_ct=(s == 14)), bound="accu")


@pytest.mark.parametrize("s", [10, 14, 18])
def test_special_values(s):
    A, B = special_inputs()
    log(f"accu special values s={s}")
    check_all_stages(A, B, s, run_stages(A, B, s), bound="accu")


def test_band_edges_and_subnormals():
    """Entries on both sides of the band edge 2^-7 (relative to the row
    maximum), exact powers of two, and rows of subnormals."""
    m, q, n = 40, 300, 33
    A, B = hpl_like(m, q, n, 1.0, seed=11)
    A[0, :] = np.ldexp(1.0, -(np.arange(q) % 16))
    A[1, :] = np.ldexp(1.0 + 2.0**-52, -(np.arange(q) % 16))
    A[2, :] = np.ldexp(1.0 - 2.0**-53, -(np.arange(q) % 16))
    A[3, :] = 2.0**-1074 * (1 + np.arange(q) % 7)
    A[4, ::3] = 2.0**-1060
    B[:, 0] = np.ldexp(1.0, -(np.arange(q) % 9)) * 0.99999
    B[:, 1] = 5e-324
    log("accu band edges")
    check_all_stages(A, B, 14, run_stages(A, B, 14), bound="accu")


def test_integer_inputs_exact():
    A, B = integer_valued(100, 64, 90, 2**10, seed=2)
    C, _ = run_dgemm(A, B, 14)
    assert np.array_equal(C, A @ B)


def test_1024_cube_full_oracle_and_dgemm():
    A, B = hpl_like(1024, 1024, 1024, 1.0, seed=0)
    log("accu 1024^3 s=14: GPU stages")
    g = run_stages(A, B, 14, want_ct=False, want_prime=True)
    Cd, _ = run_dgemm(A, B, 14)
    log("accu 1024^3 s=14: oracle")
    ref = oz.dgemm(A, B, 14, stages=True, bound="accu")
    check_all_stages(A, B, 14, g, ref=ref, bound="accu")
    assert same_doubles(Cd, ref[0]), first_diff(Cd, ref[0])


def test_longest_inner_dimension():
    """q = 2^16, the longest the int32 bound products allow."""
    q = L.OZGEMM_ACCU_Q_MAX
    A, B = hpl_like(20, q, 17, 1.0, seed=5)
    L.ozgemm_free()
    configure(64, 64, q, 14)
    L.ozgemm_set_bound(L.OZGEMM_BOUND_ACCU)
    try:
        log(f"accu q={q}")
        C, _ = run_dgemm(A, B, 14)
        g = run_stages(A, B, 14, want_ct=False, want_prime=False)
    finally:
        L.ozgemm_free()
        configure(1536, 1536, 4224, 20)
        L.ozgemm_set_bound(L.OZGEMM_BOUND_ACCU)
    ref = oz.dgemm(A, B, 14, stages=True, bound="accu")
    check_all_stages(A, B, 14, g, ref=ref, bound="accu")
    assert same_doubles(C, ref[0]), first_diff(C, ref[0])


def test_range_and_workspace_errors():
    import torch
    lib = L.lib()
    Ad = torch.zeros(8 * 70000, dtype=torch.float64, device="cuda")
    Cd = torch.zeros(64, dtype=torch.float64, device="cuda")
    L.ozgemm_free()
    configure(8, 8, 70000, 14)
    L.ozgemm_set_bound(L.OZGEMM_BOUND_ACCU)
    try:
        q = L.OZGEMM_ACCU_Q_MAX + 1
        assert lib.ozgemm_dgemm(8, 8, q, Ad.data_ptr(), 8, Ad.data_ptr(), q, Cd.data_ptr(), 8, 14) == L.OZGEMM_RANGE
        assert lib.ozgemm_dgemm(8, 8, 64, Ad.data_ptr(), 8, Ad.data_ptr(), 64, Cd.data_ptr(), 8, 1) == L.OZGEMM_RANGE
        # s_max = 2 and no room for the bound's planes in the product region
        L.ozgemm_free()
        configure(1024, 1024, 1024, 2)
        L.ozgemm_set_bound(L.OZGEMM_BOUND_ACCU)
        A = torch.zeros(1024 * 1024, dtype=torch.float64, device="cuda")
        C = torch.zeros(1024 * 1024, dtype=torch.float64, device="cuda")
        st = lib.ozgemm_dgemm(1024, 1024, 64, A.data_ptr(), 1024, A.data_ptr(), 64, C.data_ptr(), 1024, 2)
        assert st == L.OZGEMM_WORKSPACE_TOO_SMALL
    finally:
        L.ozgemm_free()
        configure(1536, 1536, 4224, 20)
        L.ozgemm_set_bound(L.OZGEMM_BOUND_ACCU)


def test_more_correct_bits_than_fast():
    A, B = hpl_like(256, 512, 256, 2.0, seed=9)
    rng = np.random.default_rng(3)
    rows, cols = rng.integers(0, 256, 200), rng.integers(0, 256, 200)
    Ca, _ = run_dgemm(A, B, 13)
    L.ozgemm_set_bound(L.OZGEMM_BOUND_FAST)
    try:
        Cf, _ = run_dgemm(A, B, 13)
    finally:
        L.ozgemm_set_bound(L.OZGEMM_BOUND_ACCU)
    from fp64_gemm_emulation_ozii_amd.accuracy import correct_bits_many
    ba = correct_bits_many(Ca[rows, cols], A, B, rows, cols)
    bf = correct_bits_many(Cf[rows, cols], A, B, rows, cols)
    log(f"accu {ba:.2f} bits vs fast {bf:.2f}")
    assert ba >= bf + 0.5
