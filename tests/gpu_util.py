"""Helpers for the GPU parity tests: move matrices to the device in the
column-major layout the C-ABI takes, run each stage entry point, and bring
every intermediate back as numpy arrays in the oracle's logical shapes."""
from __future__ import annotations

import sys

import numpy as np

from fp64_gemm_emulation_ozii_amd import ozgemm as L


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def dev_colmajor(X: np.ndarray, ld: int | None = None, fill: float = 0.0):
    """Device buffer holding X (rows x cols) column-major with leading
    dimension ld >= rows; entries of the padding rows are `fill`.  Returned as
    a (cols, ld) contiguous float64 tensor."""
    import torch
    rows, cols = X.shape
    ld = max(1, rows) if ld is None else ld
    buf = np.full((max(cols, 1), ld), fill, dtype=np.float64)
    buf[:cols, :rows] = X.T
    return torch.from_numpy(buf).cuda()


def configure(max_m: int, max_n: int, max_q: int, s_max: int = 20):
    L.ozgemm_config(s_max, max_m, max_n, max_q)


def run_stages(A: np.ndarray, B: np.ndarray, s: int, lda: int | None = None, ldb: int | None = None,
               ldc: int | None = None, want_ct: bool = True, want_prime: bool = True):
    """Run scale -> residue -> gemm -> crt through the stage entry points."""
    import torch
    m, q = A.shape
    n = B.shape[1]
    lda = lda or max(1, m)
    ldb = ldb or max(1, q)
    ldc = ldc or max(1, m)
    Ad = dev_colmajor(A, lda, fill=np.nan)
    Bd = dev_colmajor(B, ldb, fill=np.nan)
    mp, np_, qp = L.ozgemm_plane_dims(m, n, q)
    dev = "cuda"
    e = torch.full((max(m, 1),), -7, dtype=torch.int32, device=dev)
    f = torch.full((max(n, 1),), -7, dtype=torch.int32, device=dev)
    Ares = torch.full((s * mp * qp,), 99, dtype=torch.int8, device=dev)
    Bres = torch.full((s * np_ * qp,), 99, dtype=torch.int8, device=dev)
    Ap = torch.full((max(q * m, 1),), -1.0, dtype=torch.float64, device=dev) if want_prime else None
    Bp = torch.full((max(q * n, 1),), -1.0, dtype=torch.float64, device=dev) if want_prime else None
    Ct = torch.full((s * mp * np_,), 7, dtype=torch.int32, device=dev) if want_ct else None
    rt = torch.full((s * mp * np_,), 250, dtype=torch.uint8, device=dev)
    Cd = torch.full((max(n, 1), ldc), 12345.0, dtype=torch.float64, device=dev)
    L.ozgemm_stage_scale(m, n, q, s, Ad, lda, Bd, ldb, e, f)
    L.ozgemm_stage_residue(m, n, q, s, Ad, lda, Bd, ldb, e, f, Ares, Bres, Ap, Bp)
    L.ozgemm_stage_gemm(m, n, q, s, Ares, Bres, Ct, rt)
    L.ozgemm_stage_crt(m, n, q, s, rt, e, f, Cd, ldc)
    torch.cuda.synchronize()
    out = {
        "e": e.cpu().numpy()[:m],
        "f": f.cpu().numpy()[:n],
        "Ares_full": Ares.cpu().numpy().reshape(s, mp, qp),
        "Bres_full": Bres.cpu().numpy().reshape(s, np_, qp),
        "rt_full": rt.cpu().numpy().reshape(s, np_, mp),
        "C_buf": Cd.cpu().numpy(),
    }
    out["Ares"] = out["Ares_full"][:, :m, :q]
    out["Bres"] = out["Bres_full"][:, :n, :q].transpose(0, 2, 1)
    out["rt"] = out["rt_full"][:, :n, :m].transpose(0, 2, 1)
    out["C"] = out["C_buf"][:n, :m].T
    if want_ct:
        out["Ct_full"] = Ct.cpu().numpy().reshape(s, np_, mp)
        out["Ct"] = out["Ct_full"][:, :n, :m].transpose(0, 2, 1)
    if want_prime:
        out["Ap"] = Ap.cpu().numpy()[: q * m].reshape(q, m).T
        out["Bp"] = Bp.cpu().numpy()[: q * n].reshape(n, q).T
    return out


def run_dgemm(A: np.ndarray, B: np.ndarray, s: int, lda=None, ldb=None, ldc=None):
    """ozgemm_dgemm on device copies of A and B; returns C (m x n numpy)."""
    import torch
    m, q = A.shape
    n = B.shape[1]
    lda = lda or max(1, m)
    ldb = ldb or max(1, q)
    ldc = ldc or max(1, m)
    Ad = dev_colmajor(A, lda, fill=np.nan)
    Bd = dev_colmajor(B, ldb, fill=np.nan)
    Cd = torch.full((max(n, 1), ldc), 12345.0, dtype=torch.float64, device="cuda")
    L.ozgemm_dgemm(m, n, q, Ad, lda, Bd, ldb, Cd, ldc, s)
    torch.cuda.synchronize()
    buf = Cd.cpu().numpy()
    return buf[:n, :m].T, buf


def same_doubles(x: np.ndarray, y: np.ndarray) -> bool:
    """Bitwise equality, with every NaN counted equal to every NaN."""
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    if x.shape != y.shape:
        return False
    nx, ny = np.isnan(x), np.isnan(y)
    if not np.array_equal(nx, ny):
        return False
    return np.array_equal(x[~nx].view(np.uint64), y[~ny].view(np.uint64))


def within_tolerance(C: np.ndarray, Cref: np.ndarray, A: np.ndarray, B: np.ndarray) -> bool:
    """|C - Cref| <= 2^-50 (|A||B|)_ij componentwise on finite entries."""
    bound = 2.0 ** -50 * (np.abs(A) @ np.abs(B))
    fin = np.isfinite(Cref)
    if not np.array_equal(np.isnan(C), np.isnan(Cref)):
        return False
    with np.errstate(invalid="ignore"):
        return bool(np.all(np.abs(C[fin] - Cref[fin]) <= bound[fin]))


def first_diff(x, y):
    idx = np.argwhere(np.asarray(x) != np.asarray(y))
    if len(idx) == 0:
        return None
    i = tuple(idx[0])
    return i, np.asarray(x)[i], np.asarray(y)[i], len(idx)
