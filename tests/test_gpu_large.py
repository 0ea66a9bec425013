"""GPU parity at full problem sizes, in the launch configuration the
benchmark times (ozgemm_dgemm with s = 14).

Most of these are too large for the oracle as a whole, so each such test
checks (a) every row and column exponent against the oracle, and (b) a block
of output entries -- random rows and columns plus the first/last rows and
columns and rows/columns of the last output tile -- against the oracle
evaluated on exactly those rows of A and columns of B (the entries only
depend on them).  At 4096^3 the whole output is compared with the whole
oracle result, evaluated in tiles by worker processes on the host's cores.
"""
import numpy as np
import pytest

from oracle import ozaki2 as oz
from fp64_gemm_emulation_ozii_amd import ozgemm as L
from fp64_gemm_emulation_ozii_amd.synthetic import hpl_like

from gpu_util import dev_colmajor, first_diff, log, same_doubles, within_tolerance
from oracle_pool import host_workers, oracle_full

pytestmark = pytest.mark.gpu


def sample_lines(size: int, count: int, seed: int, tile: int = 256):
    rng = np.random.default_rng(seed)
    picks = set(int(v) for v in rng.integers(0, size, size=count))
    last0 = (size - 1) // tile * tile
    picks |= {0, size - 1, last0, min(size - 1, last0 + 1)}
    picks |= set(int(v) for v in rng.integers(last0, size, size=4))
    return np.array(sorted(picks), dtype=np.int64)


# parts: K parts of the product launch on a 256-CU device (1: one part; 0:
# q >= 2^17 walked as sequential K blocks, whose epilogue adds each block's
# residues to the earlier ones)
@pytest.mark.parametrize("m,q,n,phi,parts", [
    (4096, 4096, 4096, 1.0, 1),
    (8192, 8192, 8192, 1.0, 1),
    (16384, 1024, 16384, 1.0, 1),
    (16384, 384, 16384, 1.0, 1),
    (1024, 65536, 1024, 1.0, 8),
    (16384, 16384, 16384, 0.0, 1),
    (16384, 16384, 16384, 4.0, 1),
    (16384, 16384, 16384, 16.0, 1),
    (16384, 16384, 16384, 32.0, 1),
    (384, 2**20, 384, 1.0, None),
    (1792, 2**17 + 300, 1792, 1.0, 0),
])
def test_sampled_block_and_exponents(m, q, n, phi, parts):
    import torch
    s = 14
    log(f"large m={m} q={q} n={n} phi={phi}: generate")
    A, B = hpl_like(m, q, n, phi, seed=0)
    L.ozgemm_config(s, m, n, q)
    got_parts = L.ozgemm_gemm_parts(m, n, q, s)
    if parts is None:
        assert got_parts >= 16  # 2^20 / 2^16 parts at least
    else:
        assert got_parts == parts
    Ad = dev_colmajor(A)
    Bd = dev_colmajor(B)
    Cd = torch.empty((n, m), dtype=torch.float64, device="cuda")
    log("  ozgemm_dgemm")
    L.ozgemm_dgemm(m, n, q, Ad, m, Bd, q, Cd, m, s)
    e = torch.empty(m, dtype=torch.int32, device="cuda")
    f = torch.empty(n, dtype=torch.int32, device="cuda")
    L.ozgemm_stage_scale(m, n, q, s, Ad, m, Bd, q, e, f)
    torch.cuda.synchronize()
    # the oracle's cost grows with rows x cols x q: fewer lines for long K
    lines = 56 if q < 2**17 else 12
    rows = sample_lines(m, lines, seed=1)
    cols = sample_lines(n, lines, seed=2)
    Cg = Cd[torch.from_numpy(cols).cuda()][:, torch.from_numpy(rows).cuda()].cpu().numpy().T
    eg = e.cpu().numpy()
    fg = f.cpu().numpy()
    del Ad, Bd, Cd
    L.ozgemm_free()
    torch.cuda.empty_cache()
    log("  oracle exponents")
    assert np.array_equal(eg, oz.row_exponents(A))
    assert np.array_equal(fg, oz.col_exponents(B))
    log(f"  oracle block {len(rows)}x{len(cols)}")
    ref = oz.dgemm_block(A, B, s, rows, cols)
    assert within_tolerance(Cg, ref, A[rows, :], B[:, cols])
    assert same_doubles(Cg, ref)


@pytest.mark.timeout(900)
def test_full_oracle_4096_cubed():
    """4096^3, s = 14, phi = 1: every entry of C against the oracle."""
    import torch
    m = q = n = 4096
    s = 14
    log(f"full 4096^3: generate; oracle on {host_workers()} worker processes")
    A, B = hpl_like(m, q, n, 1.0, seed=0)
    L.ozgemm_config(s, m, n, q)
    Ad = dev_colmajor(A)
    Bd = dev_colmajor(B)
    Cd = torch.empty((n, m), dtype=torch.float64, device="cuda")
    L.ozgemm_dgemm(m, n, q, Ad, m, Bd, q, Cd, m, s)
    torch.cuda.synchronize()
    C = Cd.cpu().numpy().T
    del Ad, Bd, Cd
    L.ozgemm_free()
    torch.cuda.empty_cache()
    ref = oracle_full(m, q, n, 1.0, 0, s, tiles=(4, 4))
    log("  compare")
    assert same_doubles(C, ref), first_diff(C, ref)
    assert within_tolerance(C, ref, A, B)
