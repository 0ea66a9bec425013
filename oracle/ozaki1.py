"""Plain CPU oracle of Ozaki Scheme I on INT8 products (slice split).

TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py``.  Written from the
Ozaki I notes' optimized algorithms (after Uchino, Ozaki and Imamura): the
round-to-nearest split, the triangular set of slice products, the group-wise
error-free INT32 accumulation and the Hybrid split.  Matrices are logical
numpy arrays (A is m x q, B is q x n); slices are kept as integers with a
power-of-two grid exponent per row (A) or column (B).

Two variants are provided:

``rn``
    RN split of A by rows and of B by columns (Ozaki I notes, optimized
    algorithm, direction 1 and "RN split algorithm"): the grid of slice p is
    recomputed from the current residual.  Products A_i B_j for
    i + j <= k + 1 (the triangle of the basic INT algorithm), each converted
    to FP64, scaled by its two grids and added to C one at a time, i-major
    and j-minor.

``hybrid``
    Hybrid split (direction 3): the grid of the first slice is taken from the
    original row maximum and every further slice is beta bits finer.  All
    products with the same i + j then share one scale, and up to r of them
    are summed exactly in INT32 before one conversion and one FP64 addition
    (direction 2, "group-wise accumulation algorithm").

Readings taken where the notes leave a point open (also listed in the design
notes of the repository):

* beta = min(7, floor((31 - log2 q)/2)) is evaluated exactly as the largest
  b <= 7 with q 4^b <= 2^31; r = max(1, 2^(31 - 2 beta - ceil(log2 q))) with
  ceil(log2 q) taken exactly;
* E = ceil(log2 max_j |a_ij|) is exact (a power of two gives its own
  exponent); the slice grid is mu = 2^(E + 1 - beta);
* the magic-constant extraction (a + sigma) - sigma with
  sigma = 0.75 2^53 mu rounds a to the nearest multiple of mu, ties to even;
  the oracle writes that rounding as mu * rint(a / mu), which is the same
  number wherever sigma is a finite normal double and stays well defined for
  rows whose maximum is near the ends of the double range (a test evaluates
  the notes' expression literally and checks the equality);
* every one of the k slices is rounded, the last included; the residual left
  after slice k is dropped;
* the integer of a slice is the rounded value divided by its grid (the grid
  of Hybrid slice p is mu'' 2^(-beta (p-1)));
* an all-zero row (or residual row) has an all-zero slice, stored with grid
  exponent 0; a row of A or column of B holding Inf or NaN makes every
  output it touches NaN, as in the Scheme II path.
"""
from __future__ import annotations

import numpy as np

#: Grid exponent recorded for a row/column that contains Inf or NaN.
NONFINITE = 2**31 - 1


def slice_width(q: int) -> int:
    """beta = min(7, floor((31 - log2 q) / 2)) -- Ozaki I notes, algorithm
    analysis of the RN split: a signed int8 holds 7 magnitude bits, and q
    products of 2 beta bits must fit the INT32 accumulator.

    floor((31 - log2 q)/2) >= b  <=>  q <= 2^(31 - 2b)  <=>  q 4^b <= 2^31.
    """
    if q < 1:
        raise ValueError("q must be >= 1")
    b = 0
    while b < 7 and q * 4 ** (b + 1) <= 2**31:
        b += 1
    if b < 1:
        raise ValueError(f"q = {q} leaves no slice width")
    return b


def group_size(q: int, beta: int) -> int:
    """r = max(1, 2^(31 - 2 beta - ceil(log2 q))) -- Ozaki I notes, direction
    2: the number of slice products an INT32 accumulator sums exactly."""
    c = (q - 1).bit_length()  # ceil(log2 q) for q >= 1
    e = 31 - 2 * beta - c
    return max(1, 2**e) if e >= 0 else 1


def triangle(k: int) -> list[tuple[int, int]]:
    """Slice pairs (i, j), 1-based, with i + j <= k + 1, i-major and j-minor
    (Ozaki I notes, INT matrix multiplication algorithm)."""
    return [(i, j) for i in range(1, k + 1) for j in range(1, k - i + 2)]


def groups(k: int, r: int) -> list[tuple[int, list[tuple[int, int]]]]:
    """Group-wise accumulation order (Ozaki I notes, direction 2): for
    g = 2..k+1 the pairs (s, g - s), s = 1..g-1, in runs of at most r.
    Returns [(g, [pairs of one run]), ...]."""
    out = []
    for g in range(2, k + 2):
        run: list[tuple[int, int]] = []
        for s in range(1, g):
            run.append((s, g - s))
            if len(run) == r or s == g - 1:
                out.append((g, run))
                run = []
    return out


def _ceil_log2_rows(R: np.ndarray):
    """Per row: E = ceil(log2 max_j |R_ij|), plus masks of zero rows and of
    rows holding Inf/NaN."""
    R = np.asarray(R, dtype=np.float64)
    bad = ~np.all(np.isfinite(R), axis=1)
    mx = np.max(np.abs(np.where(np.isfinite(R), R, 0.0)), axis=1) if R.shape[1] else np.zeros(R.shape[0])
    zero = (mx == 0.0) & ~bad
    frac, ex = np.frexp(mx)  # mx = frac 2^ex, frac in [0.5, 1)
    E = np.where(frac == 0.5, ex - 1, ex).astype(np.int64)
    E = np.where(zero | bad, 0, E)
    return E, zero, bad


def _round_to_grid(R: np.ndarray, g: np.ndarray) -> np.ndarray:
    """Integers n = rint(R_ij / 2^g_i), ties to even (the magic-constant
    rounding of the notes), as float64 values."""
    return np.rint(np.ldexp(R, -g[:, None]))


def _residual(R: np.ndarray, n: np.ndarray, g: np.ndarray) -> np.ndarray:
    """R - n 2^g, exactly (the residual the split keeps).  Where n != 0 the
    difference is formed on the grid, (R 2^-g - n) 2^g: both steps are exact,
    and n 2^g itself may overflow when the row maximum lies within one grid
    step of the largest double.  Where n = 0 the residual is R itself."""
    with np.errstate(over="ignore", under="ignore"):
        scaled = np.ldexp(np.ldexp(R, -g[:, None]) - n, g[:, None])
    return np.where(n == 0.0, R, scaled)


def split_rn(X: np.ndarray, k: int, beta: int):
    """RN split of the rows of X into k int8 slices (Ozaki I notes, RN split
    algorithm).  Returns (slices (k, rows, cols) int8, grid exponents
    (k, rows) int64, non-finite row mask)."""
    R = np.array(X, dtype=np.float64, copy=True)
    rows, cols = R.shape
    _, _, bad = _ceil_log2_rows(R)
    R[bad, :] = 0.0
    sl = np.zeros((k, rows, cols), dtype=np.int8)
    ge = np.zeros((k, rows), dtype=np.int64)
    for p in range(k):
        E, zero, _ = _ceil_log2_rows(R)            # step 3: mu from the residual
        g = np.where(zero, 0, E + 1 - beta)        # mu = 2^(E + 1 - beta)
        n = _round_to_grid(R, g)                   # steps 4-5: (a + sigma) - sigma
        n[zero, :] = 0.0
        assert np.all(np.abs(n) <= 2 ** (beta - 1)), "slice outside int8 budget"
        sl[p] = n.astype(np.int8)                  # step 6: INT8(mu^-1 A_s)
        ge[p] = g
        R = _residual(R, n, g)                     # step 7: residual
    return sl, ge, bad


def split_hybrid(X: np.ndarray, k: int, beta: int):
    """Hybrid split of the rows of X (Ozaki I notes, Hybrid split algorithm):
    mu'' = 2^(E + 1 - beta) from the original row maximum, slice p on the grid
    mu'' 2^(-beta (p-1)).  Returns (slices (k, rows, cols) int8, exponent of
    mu'' per row, non-finite row mask)."""
    R = np.array(X, dtype=np.float64, copy=True)
    rows, cols = R.shape
    E, zero, bad = _ceil_log2_rows(R)
    R[bad, :] = 0.0
    g0 = np.where(zero | bad, 0, E + 1 - beta)
    sl = np.zeros((k, rows, cols), dtype=np.int8)
    for p in range(k):
        g = g0 - beta * p
        n = _round_to_grid(R, g)
        n[zero | bad, :] = 0.0
        assert np.all(np.abs(n) <= 2 ** (beta - 1)), "slice outside int8 budget"
        sl[p] = n.astype(np.int8)
        R = _residual(R, n, g)
    return sl, g0.astype(np.int64), bad


def int_product(Asl: np.ndarray, Bsl: np.ndarray) -> np.ndarray:
    """Exact integer product of an A slice (m x q) and a B slice (q x n)."""
    P = Asl.astype(np.int64) @ Bsl.astype(np.int64)
    assert np.all(np.abs(P) < 2**31), "INT32 accumulator overflow"
    return P


def dgemm_rn(A: np.ndarray, B: np.ndarray, k: int, stages: bool = False):
    """C ~ AB by the RN split and triangular products with per-product FP64
    accumulation, i-major, j-minor (Ozaki I notes, direction 1 with the INT
    matrix multiplication algorithm)."""
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    m, q = A.shape
    n = B.shape[1]
    beta = slice_width(max(q, 1))
    As, gA, badA = split_rn(A, k, beta)
    Bs_t, gB, badB = split_rn(B.T, k, beta)      # columns of B as rows
    Bs = np.transpose(Bs_t, (0, 2, 1))
    C = np.zeros((m, n))
    prods = []
    for i, j in triangle(k):
        P = int_product(As[i - 1], Bs[j - 1])
        term = np.ldexp(P.astype(np.float64), gA[i - 1][:, None] + gB[j - 1][None, :])
        C = C + term
        prods.append(P)
    C[badA, :] = np.nan
    C[:, badB] = np.nan
    if not stages:
        return C
    return C, {"beta": beta, "As": As, "Bs": Bs, "gA": gA, "gB": gB, "pairs": triangle(k),
               "products": prods, "C": C}


def dgemm_hybrid(A: np.ndarray, B: np.ndarray, k: int, stages: bool = False):
    """C ~ AB by the Hybrid split and group-wise error-free accumulation
    (Ozaki I notes, directions 2 and 3): runs of at most r products with the
    same i + j = g are summed in INT32, then scaled by
    mu''_i nu''_j 2^(-beta (g - 2)) and added to C in FP64."""
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    m, q = A.shape
    n = B.shape[1]
    beta = slice_width(max(q, 1))
    r = group_size(max(q, 1), beta)
    As, gA, badA = split_hybrid(A, k, beta)
    Bs_t, gB, badB = split_hybrid(B.T, k, beta)
    Bs = np.transpose(Bs_t, (0, 2, 1))
    C = np.zeros((m, n))
    sums = []
    order = groups(k, r)
    for g, run in order:
        P = np.zeros((m, n), dtype=np.int64)
        for s, t in run:
            P = P + int_product(As[s - 1], Bs[t - 1])
        assert np.all(np.abs(P) < 2**31), "INT32 group accumulator overflow"
        term = np.ldexp(P.astype(np.float64), gA[:, None] + gB[None, :] - beta * (g - 2))
        C = C + term
        sums.append(P)
    C[badA, :] = np.nan
    C[:, badB] = np.nan
    if not stages:
        return C
    return C, {"beta": beta, "r": r, "As": As, "Bs": Bs, "gA": gA, "gB": gB, "groups": order,
               "products": sums, "C": C}


def dgemm(A, B, k: int, variant: str = "rn", stages: bool = False):
    if variant == "rn":
        return dgemm_rn(A, B, k, stages)
    if variant == "hybrid":
        return dgemm_hybrid(A, B, k, stages)
    raise ValueError(f"unknown variant {variant!r}")
