"""ozgemm_dgemm captured into a HIP graph.

After one call outside capture (which uploads the CRT constant table), a
call only enqueues kernels on the configured stream, so it can be captured.
Each graph is replayed several times with other eager GPU work and
synchronisations between the replays, and every replay must reproduce the
eager result bit for bit.  The shapes cover the persistent product grid
with K parts and the parts' reduction, both wavefront counts of the product
kernel, a long inner dimension, and the one-pass residue kernel of B.
"""
import numpy as np
import pytest

from fp64_gemm_emulation_ozii_amd import ozgemm as L
from fp64_gemm_emulation_ozii_amd.synthetic import hpl_like

from gpu_util import dev_colmajor, log

pytestmark = pytest.mark.gpu


# 768 x 65536 x 512: 12 K parts, 1008 blocks on the persistent grid (four
# wavefronts), then the parts' reduction; 1536 x 1024 x 1536: persistent
# grid, one part, eight wavefronts; 900 x 300 x 1300: three K slices (eight
# wavefronts); 300 x (2^17 + 300) x 200: long K as parts; 1024 x 5000 x 700:
# B's exponents taken in its residue pass (ragged K), one block per tile
@pytest.mark.parametrize("m,q,n,s", [(768, 65536, 512, 14), (1536, 1024, 1536, 14), (900, 300, 1300, 14),
                                     (300, 2**17 + 300, 200, 12), (1024, 5000, 700, 14)])
def test_dgemm_replays_from_a_graph(m, q, n, s):
    import torch
    A, B = hpl_like(m, q, n, 1.0, seed=m + n)
    stream = torch.cuda.Stream()
    L.ozgemm_free()
    L.ozgemm_config(s, m, n, q, stream=stream)
    try:
        log(f"graph m={m} q={q} n={n} s={s} parts={L.ozgemm_gemm_parts(m, n, q, s)}")
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
            Y = X @ X  # eager work between the replays
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            got = C_graph.cpu().numpy()
            assert np.array_equal(got.view(np.uint64), want.view(np.uint64)), f"replay {rep}"
            assert torch.isfinite(Y).all()
        del graph
    finally:
        L.ozgemm_free()
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
