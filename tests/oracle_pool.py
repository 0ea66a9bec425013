"""The oracle on a whole large output, cut into tiles that worker processes
evaluate in parallel on the host's cores.

Each worker regenerates the seeded inputs (fp64_gemm_emulation_ozii_amd.
synthetic.hpl_like) and runs ``oracle.ozaki2.dgemm_block`` on its tile of
rows x columns.  A tile of the oracle equals the same entries of the full
oracle result, because the exponents depend only on their own row of A or
column of B and k only on q (pinned by
test_oracle_pins.py::test_block_entries_equal_full_entries).  Workers are
fresh interpreters (the "spawn" start method): they never touch a GPU, and
their BLAS runs single-threaded.
"""
from __future__ import annotations

import os

import numpy as np


def _tile(job):
    from oracle import ozaki2 as oz
    from fp64_gemm_emulation_ozii_amd.synthetic import hpl_like
    (m, q, n, phi, seed), s, bound, r0, r1, c0, c1 = job
    A, B = hpl_like(m, q, n, phi, seed=seed)
    return r0, c0, oz.dgemm_block(A, B, s, np.arange(r0, r1), np.arange(c0, c1), bound=bound)


def host_workers(cap: int = 16) -> int:
    try:
        cpus = len(os.sched_getaffinity(0))
    except AttributeError:
        cpus = os.cpu_count() or 1
    return max(1, min(cap, cpus))


def oracle_full(m: int, q: int, n: int, phi: float, seed: int, s: int, tiles: tuple[int, int] = (4, 4),
                bound: str = "conservative", workers: int = 0, timeout: float = 900.0) -> np.ndarray:
    """The oracle's m x n result for hpl_like(m, q, n, phi, seed), computed as
    tiles[0] x tiles[1] blocks in a pool of worker processes."""
    import multiprocessing as mp
    W = workers if workers > 0 else host_workers()
    rb = np.linspace(0, m, tiles[0] + 1).astype(int)
    cb = np.linspace(0, n, tiles[1] + 1).astype(int)
    jobs = [((m, q, n, phi, seed), s, bound, int(rb[i]), int(rb[i + 1]), int(cb[j]), int(cb[j + 1]))
            for i in range(tiles[0]) for j in range(tiles[1])]
    env = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")
    saved = {k: os.environ.get(k) for k in env}
    for k in env:
        os.environ[k] = "1"
    try:
        with mp.get_context("spawn").Pool(W) as pool:
            parts = pool.map_async(_tile, jobs, chunksize=1).get(timeout=timeout)
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    C = np.empty((m, n), dtype=np.float64)
    for r0, c0, blk in parts:
        C[r0:r0 + blk.shape[0], c0:c0 + blk.shape[1]] = blk
    return C
