"""The product stage at the ends of the int32 range, in every grid form.

ozgemm_stage_gemm runs on residue planes built here with constant rows and
columns: row i of plane t of A holds x_t[i] at every K index below q, and
column j of B holds y_t[j].  The exact product is then C_t[i, j] =
q x_t[i] y_t[j], and its residue is that integer's floor-mod by m_t -- a
closed form evaluated in numpy int64, independent of the GPU path.  Row 0 of
A and column 0 of B hold -128, row 1 and column 1 hold 127, so C_t[0, 0] =
q 2^14 and C_t[0, 1] = -q 128 127 are the largest and most negative entries
any int8 product of this length can reach; the rest are random int8 values.
At q = 130944 (the longest K one launch sums) C_t[0, 0] is 2^31 - 2^21, which
with the residue-only kernels' accumulator start of -(m_t - 1)/2 is the
largest accumulator the epilogue sees.

Cases, one per grid form of the product launch (the form is named in the
log line; the split choice is also checked through ozgemm_gemm_parts):
  * persistent form, one K part: 4096 x 2304 x 130944, s = 14;
  * sequential K blocks (q >= 2^17 and a workspace too small for two K
    parts' planes): 4096 x 2304 x (2^17 + 300), s = 14;
  * K parts: 256 x 256 x 130907 (16 parts, ragged K), s = 14;
  * one block per tile, eight wavefronts per block (at most 16 K slices):
    256 x 256 x 640, s = 14;
  * persistent form with eight wavefronts: 2048 x 2048 x 512 and
    2048 x 2048 x 500, s = 14;
  * int32 planes and residues together (the unbiased debug form):
    512 x 512 x 130944, s = 14, both outputs checked.
"""
import numpy as np
import pytest

from oracle import ozaki2 as oz
from fp64_gemm_emulation_ozii_amd import ozgemm as L

from gpu_util import first_diff, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu_present():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    yield
    L.ozgemm_free()
    torch.cuda.empty_cache()


def extreme_values(count: int, s: int, rng: np.random.Generator, third: int) -> np.ndarray:
    v = rng.integers(-128, 128, size=(s, count), dtype=np.int64)
    v[:, 0] = -128
    if count > 1:
        v[:, 1] = 127
    if count > 2:
        v[:, 2] = third
    return v


def run_case(m, n, q, s, want_ct=False, seed=0):
    """Build the planes on the device, run the product stage, and compare
    with the closed form.  Returns the K parts the library chose."""
    import torch
    rng = np.random.default_rng(seed)
    x = extreme_values(m, s, rng, 0)
    y = extreme_values(n, s, rng, 1)
    L.ozgemm_free()
    torch.cuda.empty_cache()
    L.ozgemm_config(s, m, n, q)
    try:
        parts = L.ozgemm_gemm_parts(m, n, q, s)
        mp, np_, qp = L.ozgemm_plane_dims(m, n, q)
        Ares = torch.zeros((s, mp, qp), dtype=torch.int8, device="cuda")
        Bres = torch.zeros((s, np_, qp), dtype=torch.int8, device="cuda")
        Ares[:, :m, :q] = torch.from_numpy(x.astype(np.int8)).to("cuda")[:, :, None]
        Bres[:, :n, :q] = torch.from_numpy(y.astype(np.int8)).to("cuda")[:, :, None]
        rt = torch.full((s, np_, mp), 250, dtype=torch.uint8, device="cuda")
        Ct = torch.full((s, np_, mp), 7, dtype=torch.int32, device="cuda") if want_ct else None
        L.ozgemm_stage_gemm(m, n, q, s, Ares, Bres, Ct, rt)
        torch.cuda.synchronize()
        del Ares, Bres
        rt_h = rt.cpu().numpy()
        ct_h = Ct.cpu().numpy() if want_ct else None
    finally:
        L.ozgemm_free()
        torch.cuda.empty_cache()
    moduli = oz.greedy_moduli(s)
    for t in range(s):
        C = q * np.outer(x[t], y[t])  # exact: |C| < 2^31
        want = np.mod(C, moduli[t]).T  # stored column-major: [j, i]
        got = rt_h[t, :n, :m]
        assert np.array_equal(got, want), f"plane {t} (m_t = {moduli[t]}): {first_diff(got, want)}"
        if want_ct:
            assert np.array_equal(ct_h[t, :n, :m], C.T), f"int32 plane {t}: {first_diff(ct_h[t, :n, :m], C.T)}"
    return parts


def test_extremes_persistent_single_part():
    m, n, q, s = 4096, 2304, 130944, 14
    log(f"extremes, persistent form: {m} x {n} x {q}, s = {s}")
    assert run_case(m, n, q, s, seed=1) <= 1


def test_extremes_sequential_k_blocks():
    m, n, q, s = 4096, 2304, 2**17 + 300, 14
    log(f"extremes, sequential K blocks: {m} x {n} x {q}, s = {s}")
    assert run_case(m, n, q, s, seed=2) <= 1


def test_extremes_k_parts():
    m, n, q, s = 256, 256, 130907, 14
    log(f"extremes, K parts: {m} x {n} x {q}, s = {s}")
    assert run_case(m, n, q, s, seed=3) == 16


def test_extremes_block_per_tile():
    m, n, q, s = 256, 256, 640, 14
    log(f"extremes, one block per tile, eight wavefronts: {m} x {n} x {q}, s = {s}")
    assert run_case(m, n, q, s, seed=4) <= 1


@pytest.mark.parametrize("q", [512, 500])
def test_extremes_short_k(q):
    m, n, s = 2048, 2048, 14
    log(f"extremes, persistent form, eight wavefronts: {m} x {n} x {q}, s = {s}")
    assert run_case(m, n, q, s, seed=5 + q) <= 1


def test_extremes_int32_planes_and_residues():
    m, n, q, s = 512, 512, 130944, 14
    log(f"extremes, int32 planes + residues: {m} x {n} x {q}, s = {s}")
    run_case(m, n, q, s, want_ct=True, seed=6)
