"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle checks.

This module holds no arithmetic of the emulation method: it only draws input
matrices.  The Ozaki Scheme II notes (chatdocs.ruinique.com/nla/ozaki-scheme-ii,
§10) measure accuracy on "HPL-like" data with a dynamic-range knob phi; the
generator below is that family:

    a = (U(0,1) - 0.5) * exp(phi * N(0,1))

Entries have a uniform random sign and a log-normal magnitude whose spread
grows with phi.  A is drawn first (m x q), then B (q x n), from one
``numpy.random.default_rng(seed)`` stream, each as uniform draws followed by
normal draws.  Both are returned in Fortran (column-major) order, the layout
the C-ABI takes.
"""
from __future__ import annotations

import numpy as np


def hpl_like(m: int, q: int, n: int, phi: float, seed: int = 0):
    """Return (A, B) with A m x q and B q x n, float64, column-major."""
    rng = np.random.default_rng(seed)
    A = (rng.random((m, q)) - 0.5) * np.exp(phi * rng.standard_normal((m, q)))
    B = (rng.random((q, n)) - 0.5) * np.exp(phi * rng.standard_normal((q, n)))
    return np.asfortranarray(A), np.asfortranarray(B)


def integer_valued(m: int, q: int, n: int, bound: int, seed: int = 0):
    """Integer-valued float64 matrices with entries in [-bound, bound]."""
    rng = np.random.default_rng(seed)
    A = rng.integers(-bound, bound + 1, size=(m, q)).astype(np.float64)
    B = rng.integers(-bound, bound + 1, size=(q, n)).astype(np.float64)
    return np.asfortranarray(A), np.asfortranarray(B)


def sample_entries(m: int, n: int, count: int, seed: int = 12345, tile: int = 64):
    """Output positions to check on large problems.

    ``count`` uniform (i, j) pairs, plus the four corners and up to 32 entries
    inside the last (possibly partial) output tile.  Returns two int64 arrays.
    """
    rng = np.random.default_rng(seed)
    rows = list(rng.integers(0, m, size=count))
    cols = list(rng.integers(0, n, size=count))
    rows += [0, m - 1, 0, m - 1]
    cols += [0, n - 1, n - 1, 0]
    r0 = (m - 1) // tile * tile
    c0 = (n - 1) // tile * tile
    rows += list(rng.integers(r0, m, size=32))
    cols += list(rng.integers(c0, n, size=32))
    return np.asarray(rows, dtype=np.int64), np.asarray(cols, dtype=np.int64)
