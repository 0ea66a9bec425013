"""ozgemm_dgemm_noalloc: the entry point for callers that cannot allocate.

It must give the same result as ozgemm_dgemm (same kernels, intermediates in
the library's fixed device array instead of the configured workspace), bit
for bit, on calls in a row whose sizes shrink (the array keeps the previous
call's contents), under each of the three bit budgets; it refuses shapes
whose intermediates exceed the array.
"""
import numpy as np
import pytest

from oracle import ozaki2 as oz
from fp64_gemm_emulation_ozii_amd import ozgemm as L
from fp64_gemm_emulation_ozii_amd.synthetic import hpl_like

from gpu_util import dev_colmajor, first_diff, log, same_doubles, within_tolerance

pytestmark = pytest.mark.gpu


def both(A, B, s, stream):
    """C from ozgemm_dgemm (configured workspace) and from
    ozgemm_dgemm_noalloc, through the C-ABI."""
    import torch
    m, q = A.shape
    n = B.shape[1]
    Ad = dev_colmajor(A, m + 3, fill=np.nan)
    Bd = dev_colmajor(B, q + 1, fill=np.nan)
    C1 = torch.full((n, m + 2), 7.0, dtype=torch.float64, device="cuda")
    C2 = torch.full((n, m + 2), -7.0, dtype=torch.float64, device="cuda")
    L.ozgemm_dgemm(m, n, q, Ad, m + 3, Bd, q + 1, C1, m + 2, s)
    st = L.lib().ozgemm_dgemm_noalloc(m, n, q, Ad.data_ptr(), m + 3, Bd.data_ptr(), q + 1, C2.data_ptr(), m + 2, s,
                                      stream.cuda_stream)
    assert st == 0, L.ozgemm_strerror(st)
    torch.cuda.synchronize()
    c1, c2 = C1.cpu().numpy(), C2.cpu().numpy()
    assert np.all(c2[:, m:] == -7.0), "ldc padding written"
    return c1[:n, :m].T, c2[:n, :m].T


BOUND_NAMES = {L.OZGEMM_BOUND_CONSERVATIVE: "conservative", L.OZGEMM_BOUND_FAST: "fast",
               L.OZGEMM_BOUND_ACCU: "accu"}


@pytest.mark.parametrize("bound", [L.OZGEMM_BOUND_CONSERVATIVE, L.OZGEMM_BOUND_FAST, L.OZGEMM_BOUND_ACCU])
def test_noalloc_matches_dgemm_on_shrinking_calls(bound):
    import torch
    stream = torch.cuda.Stream()
    L.ozgemm_config(16, 1100, 1000, 4200)
    L.ozgemm_set_bound(bound)
    try:
        for (m, n, q, s, phi) in [(1100, 1000, 2100, 16, 1.0), (300, 257, 129, 14, 0.5), (65, 33, 4097, 12, 2.0)]:
            log(f"noalloc bound={bound} m={m} n={n} q={q} s={s}")
            A, B = hpl_like(m, q, n, phi, seed=m + q)
            A[3, :] = 0.0
            B[:, 5] *= 2.0**-1030
            with torch.cuda.stream(stream):
                c1, c2 = both(A, B, s, stream)
            assert same_doubles(c1, c2), first_diff(c1, c2)
            if m * n * q <= 300 * 257 * 129:
                ref = oz.dgemm(A, B, s, bound=BOUND_NAMES[bound])
                assert same_doubles(c2, ref), first_diff(c2, ref)
                assert within_tolerance(c2, ref, A, B)
    finally:
        L.ozgemm_set_bound(L.OZGEMM_BOUND_CONSERVATIVE)
        L.ozgemm_free()


def test_noalloc_empty_zero_q_and_range():
    import torch
    lib = L.lib()
    L.ozgemm_free()  # no configuration is needed
    A = torch.ones((8, 8), dtype=torch.float64, device="cuda")
    C = torch.full((8, 8), 5.0, dtype=torch.float64, device="cuda")
    assert lib.ozgemm_dgemm_noalloc(8, 8, 0, A.data_ptr(), 8, A.data_ptr(), 1, C.data_ptr(), 8, 14, None) == 0
    torch.cuda.synchronize()
    assert np.all(C.cpu().numpy() == 0.0)
    assert lib.ozgemm_dgemm_noalloc(0, 8, 8, A.data_ptr(), 1, A.data_ptr(), 8, C.data_ptr(), 1, 14, None) == 0
    assert lib.ozgemm_dgemm_noalloc(8, 8, 8, A.data_ptr(), 8, A.data_ptr(), 8, C.data_ptr(), 8, 0, None) == -10
    # 4096 x 4096 x 4096 at s = 14 needs about 700 MB of intermediates
    big = 4096
    assert L.ozgemm_workspace_bytes(big, big, big, 14) > L.OZGEMM_NOALLOC_BYTES
    assert lib.ozgemm_dgemm_noalloc(big, big, big, A.data_ptr(), big, A.data_ptr() + (1 << 30), big,
                                    C.data_ptr() + (1 << 31), big, 14, None) == L.OZGEMM_RANGE
    # the largest documented fit
    assert L.ozgemm_workspace_bytes(2048, 2048, 1024, 14) <= L.OZGEMM_NOALLOC_BYTES
    assert L.ozgemm_workspace_bytes(1024, 1024, 1024, 20) <= L.OZGEMM_NOALLOC_BYTES
