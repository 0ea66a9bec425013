"""FP64 GEMM emulated with exact int8 matrix-core products (Ozaki Scheme II)
on AMD MI355X.

The computation lives in the HIP library ``libozgemm.so`` (C-ABI in
``include/ozgemm.h``); :mod:`.ozgemm` is its ctypes binding and
:mod:`.synthetic` draws seeded inputs.  Importing the package loads nothing;
the library is opened on first use and its absence is an error.
"""
from . import ozgemm  # noqa: F401
from .ozgemm import OzgemmError  # noqa: F401

__all__ = ["ozgemm", "OzgemmError", "dgemm_colmajor"]


def dgemm_colmajor(A_cm, B_cm, m: int, n: int, q: int, s: int, C_cm=None):
    """C = A B for column-major device buffers given as torch tensors.

    ``A_cm`` holds A (m x q) column-major with lda = m (for instance the
    contiguous tensor ``A.t().contiguous()``), ``B_cm`` holds B (q x n) with
    ldb = q.  Returns ``C_cm`` (n x m tensor whose memory is C column-major,
    ldc = m).  The library must be configured.
    """
    import torch
    if C_cm is None:
        C_cm = torch.empty((n, m), dtype=torch.float64, device=A_cm.device)
    ozgemm.ozgemm_dgemm(m, n, q, A_cm, max(1, m), B_cm, max(1, q), C_cm, max(1, m), s)
    return C_cm
