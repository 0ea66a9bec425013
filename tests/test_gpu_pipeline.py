"""The column-panel pipeline of ozgemm_dgemm (ozgemm_set_panels): the CRT of
panel p runs on the library's second stream while panel p + 1's product
runs.  Results must equal the unpipelined call
and the oracle bit for bit, under every bit budget, with ragged last panels
and B's one-pass residues, and a pipelined call must replay from a HIP graph
(the second stream forks from and joins back to the captured stream)."""
import numpy as np
import pytest

from oracle import ozaki2 as oz
from fp64_gemm_emulation_ozii_amd import ozgemm as L
from fp64_gemm_emulation_ozii_amd.synthetic import hpl_like

from gpu_util import dev_colmajor, first_diff, log, same_doubles
from test_gpu_parity import special_inputs

pytestmark = pytest.mark.gpu

BOUNDS = {"conservative": L.OZGEMM_BOUND_CONSERVATIVE, "fast": L.OZGEMM_BOUND_FAST, "accu": L.OZGEMM_BOUND_ACCU}


def dgemm_panels(A, B, s, panels, bound="conservative", ldc_extra=3):
    import torch
    m, q = A.shape
    n = B.shape[1]
    L.ozgemm_set_bound(BOUNDS[bound])
    L.ozgemm_set_panels(panels)
    try:
        Ad = dev_colmajor(A, m + 1, fill=np.nan)
        Bd = dev_colmajor(B, q + 2, fill=np.nan)
        Cd = torch.full((n, m + ldc_extra), 77.0, dtype=torch.float64, device="cuda")
        L.ozgemm_dgemm(m, n, q, Ad, m + 1, Bd, q + 2, Cd, m + ldc_extra, s)
        torch.cuda.synchronize()
        buf = Cd.cpu().numpy()
    finally:
        L.ozgemm_set_panels(0)
        L.ozgemm_set_bound(L.OZGEMM_BOUND_CONSERVATIVE)
    assert np.all(buf[:, m:] == 77.0), "ldc padding written"
    return buf[:, :m].T


@pytest.fixture(scope="module", autouse=True)
def config():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    L.ozgemm_config(15, 1100, 1700, 4300)
    yield
    L.ozgemm_free()


@pytest.mark.parametrize("m,q,n,s,panels", [(300, 770, 1000, 14, 3), (513, 700, 1700, 12, 4), (129, 128, 600, 15, 2),
                                            (1100, 4100, 1300, 14, 5), (64, 1000, 257, 8, 2)])
@pytest.mark.parametrize("bound", ["conservative", "fast", "accu"])
def test_pipelined_equals_unpipelined_and_oracle(m, q, n, s, panels, bound):
    A, B = hpl_like(m, q, n, 1.0, seed=m + q + n)
    log(f"pipeline {bound} m={m} q={q} n={n} s={s} panels={panels}")
    Cp = dgemm_panels(A, B, s, panels, bound)
    C1 = dgemm_panels(A, B, s, 1, bound)
    assert same_doubles(Cp, C1), first_diff(Cp, C1)
    if m * n * q <= 300 * 1000 * 770 and bound != "accu":
        rows = np.arange(0, m, 7)
        cols = np.concatenate([np.arange(0, n, 11), [n - 1]])
        ref = oz.dgemm_block(A, B, s, rows, cols, bound=bound)
        assert same_doubles(Cp[np.ix_(rows, cols)], ref)
    elif bound == "accu" and m * n * q <= 300 * 1000 * 770:
        ref = oz.dgemm(A, B, s, bound="accu")
        assert same_doubles(Cp, ref), first_diff(Cp, ref)


def test_pipelined_special_values():
    A, B = special_inputs()
    B = np.concatenate([B] * 9, axis=1)  # 594 columns: three panels of 256
    log("pipeline special values")
    Cp = dgemm_panels(A, B, 14, 3)
    ref = oz.dgemm(A, B, 14)
    assert same_doubles(Cp, ref), first_diff(Cp, ref)


def test_settings():
    assert L.lib().ozgemm_set_panels(-1) == -1
    assert L.lib().ozgemm_set_panels(L.OZGEMM_PANELS_MAX + 1) == -1
    assert L.ozgemm_set_panels(L.OZGEMM_PANELS_MAX) == 0
    assert L.ozgemm_set_panels(0) == 0


@pytest.mark.parametrize("m,q,n,s,panels", [(1024, 1024, 1300, 14, 4), (700, 5000, 900, 14, 3)])
def test_pipelined_call_replays_from_a_graph(m, q, n, s, panels):
    import torch
    A, B = hpl_like(m, q, n, 1.0, seed=m + n)
    stream = torch.cuda.Stream()
    L.ozgemm_free()
    L.ozgemm_config(s, m, n, q, stream=stream)
    L.ozgemm_set_panels(panels)
    try:
        log(f"pipeline graph m={m} q={q} n={n} panels={panels}")
        Ad, Bd = dev_colmajor(A), dev_colmajor(B)
        C_eager = torch.empty((n, m), dtype=torch.float64, device="cuda")
        C_graph = torch.empty((n, m), dtype=torch.float64, device="cuda")
        with torch.cuda.stream(stream):
            L.ozgemm_dgemm(m, n, q, Ad, m, Bd, q, C_eager, m, s)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            L.ozgemm_dgemm(m, n, q, Ad, m, Bd, q, C_graph, m, s)
        torch.cuda.synchronize()
        want = C_eager.cpu().numpy()
        X = torch.randn(512, 512, dtype=torch.float32, device="cuda")
        for rep in range(3):
            C_graph.fill_(float("nan"))
            Y = X @ X
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            got = C_graph.cpu().numpy()
            assert np.array_equal(got.view(np.uint64), want.view(np.uint64)), f"replay {rep}"
            assert torch.isfinite(Y).all()
        del graph
        L.ozgemm_set_panels(1)
        C1 = torch.empty((n, m), dtype=torch.float64, device="cuda")
        with torch.cuda.stream(stream):
            L.ozgemm_dgemm(m, n, q, Ad, m, Bd, q, C1, m, s)
        torch.cuda.synchronize()
        assert np.array_equal(C1.cpu().numpy().view(np.uint64), want.view(np.uint64))
    finally:
        L.ozgemm_set_panels(0)
        L.ozgemm_free()
        L.ozgemm_config(15, 1100, 1700, 4300)
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
