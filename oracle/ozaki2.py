"""Plain CPU oracle of Ozaki Scheme II (FP64 GEMM from exact INT8 GEMMs + CRT).

TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py``.  Slow on purpose:
every step is written the way the Ozaki II notes state it, in exact integer
arithmetic (Python ``int``) or in float64 operations that are exact for the
values they see.  Matrices here are logical numpy arrays (A is m x q, B is
q x n); memory layout plays no part.

Pipeline, in the notes' order (Ozaki II notes §7, "Algorithm 1"):

  step 1  bit budget k from M = prod(m_t) and q           -> :func:`kbits`
  step 2  power-of-two scaling D, E and truncation        -> :func:`row_exponents`,
          A' = trunc(DA), B' = trunc(BE)                      :func:`truncate_rows`
  step 3  per modulus: symmetric residues, one exact       -> :func:`smod`,
          integer product, re-reduction of the product        :func:`residue_product`,
                                                              :func:`reduce_product`
  step 4  CRT accumulation Z = sum_t C''_t M_t y_t         -> :func:`crt_combine`
  step 5  range reduction to the symmetric representative -> :func:`crt_combine`
  step 6  unscaling C = D^-1 C''' E^-1                     -> :func:`unscale`

Readings taken where the notes leave a choice open (each one also listed with
its reason in the design notes of the repository):

* moduli: the greedy pairwise-coprime sequence from 256 downward
  (256, 255, 253, 251, 247, ...); the notes only require pairwise coprime
  moduli in [2, 256] (§4, §6);
* exponents: e_i is the frexp exponent of max_l |a_il|, i.e. 2^(e_i-1) <=
  max < 2^e_i, so |a_il * 2^(k-e_i)| < 2^k; D = diag(2^(k-e_i)) (§3, §5);
* truncation is toward zero (§3, §7 step 2);
* k_A = k_B = k, the notes' equal-precision choice (§5), evaluated with exact
  integers;
* symmetric residue range for modulus m is [-floor(m/2), ceil(m/2) - 1],
  which is [-128, 127] for m = 256 (§6);
* C_t mod m_t takes the non-negative representative (§4, §7 step 3);
* the final FP64 value is X * 2^(e_i + f_j - 2k) rounded once to nearest-even,
  including the subnormal and overflow ranges (§7 step 6);
* a row of A or column of B holding Inf or NaN gets the exponent sentinel
  ``NONFINITE``; its integer row/column is zero and every output it touches
  is NaN.  An all-zero row/column has exponent 0 (frexp of 0.0) and yields +0.
"""
from __future__ import annotations

import math

import numpy as np

#: Exponent recorded for a row/column that contains Inf or NaN.
NONFINITE = 2**31 - 1

#: Largest modulus usable with signed int8 residues (Ozaki II notes §6).
MODULUS_MAX = 256


# ----------------------------------------------------------------------------
# Step 1: moduli, CRT constants, bit budget
# ----------------------------------------------------------------------------

def greedy_moduli(s: int) -> list[int]:
    """First ``s`` moduli: scan 256, 255, ... and keep each candidate that is
    coprime to every modulus already kept.

    Ozaki II notes §4 require pairwise-coprime moduli; §6 bounds them by
    2 <= m_t <= 256 so that symmetric residues fit in int8.
    """
    if s < 1:
        raise ValueError("s must be >= 1")
    chosen: list[int] = []
    cand = MODULUS_MAX
    while len(chosen) < s:
        if cand < 2:
            raise ValueError(f"fewer than {s} pairwise-coprime moduli in [2, 256]")
        if all(math.gcd(cand, c) == 1 for c in chosen):
            chosen.append(cand)
        cand -= 1
    return chosen


def crt_constants(moduli: list[int]):
    """M = prod m_t, M_t = M / m_t and y_t = M_t^-1 mod m_t (Ozaki II notes §4).

    Returns ``(M, Mt, yt)`` with Python integers; y_t is the representative in
    [0, m_t).
    """
    M = 1
    for m in moduli:
        M *= m
    Mt = [M // m for m in moduli]
    yt = [pow(Mt_t % m, -1, m) for Mt_t, m in zip(Mt, moduli)]
    return M, Mt, yt


def kbits(M: int, q: int) -> int:
    """k = floor(1/2 * log2((M/2 - 1) / q)), evaluated exactly (Ozaki II notes §5).

    floor(log2(x)) for x = (M/2 - 1)/q is the largest integer j with
    q * 2^j <= M/2 - 1, i.e. 2q * 2^j <= M - 2.  For j >= 0 it equals the bit
    length of floor((M - 2) / (2q)) minus one.  Returns a value < 1 when the
    budget leaves no bits (the caller must then reject the problem).
    """
    if q < 1:
        raise ValueError("q must be >= 1")
    t = (M - 2) // (2 * q)
    if t < 1:
        return -1
    j = t.bit_length() - 1
    return j // 2


# ----------------------------------------------------------------------------
# Step 2: exponents and truncation
# ----------------------------------------------------------------------------

def row_exponents(A: np.ndarray) -> np.ndarray:
    """e_i with 2^(e_i - 1) <= max_l |a_il| < 2^e_i (frexp exponent), int32.

    All-zero rows get 0; rows holding Inf/NaN get ``NONFINITE``.
    (Ozaki II notes §3: D has power-of-two diagonal entries; §5: the bound
    c_max <= q 2^(k_A+k_B) needs |DA| < 2^k_A.)
    """
    A = np.asarray(A, dtype=np.float64)
    e = np.zeros(A.shape[0], dtype=np.int64)
    if A.shape[1] == 0:
        return e.astype(np.int32)
    amax = np.max(np.abs(A), axis=1)
    for i, v in enumerate(amax):
        v = float(v)
        if not math.isfinite(v):
            e[i] = NONFINITE
        else:
            e[i] = math.frexp(v)[1]
    return e.astype(np.int32)


def col_exponents(B: np.ndarray) -> np.ndarray:
    """f_j, the exponent of column j of B (same rule as :func:`row_exponents`)."""
    return row_exponents(np.asarray(B).T)


def truncate_rows(A: np.ndarray, e: np.ndarray, k: int) -> np.ndarray:
    """A' = trunc(D A) with D = diag(2^(k - e_i)) (Ozaki II notes §3, §7 step 2).

    Returned as float64 holding exact integers (|A'| <= 2^k - 1, at most 53
    significant bits).  Multiplying by a power of two is exact unless the
    product drops below 2^-1022; such products are below 1 in magnitude and
    truncate to 0 either way, so trunc(ldexp(a, k - e_i)) is exact.  Rows with
    the ``NONFINITE`` sentinel are zero.  -0.0 is normalised to +0.0.
    """
    A = np.asarray(A, dtype=np.float64)
    e64 = np.asarray(e, dtype=np.int64)
    bad = e64 == NONFINITE
    shift = np.where(bad, 0, k - e64).astype(np.int32)
    Ap = np.trunc(np.ldexp(A, shift[:, None]))
    Ap[bad, :] = 0.0
    return Ap + 0.0


def truncate_cols(B: np.ndarray, f: np.ndarray, k: int) -> np.ndarray:
    """B' = trunc(B E) with E = diag(2^(k - f_j))."""
    return truncate_rows(np.asarray(B).T, f, k).T


# ----------------------------------------------------------------------------
# Step 3: symmetric residues, exact products, re-reduction
# ----------------------------------------------------------------------------

def smod(X: np.ndarray, m: int) -> np.ndarray:
    """Symmetric residue of integer-valued float64 X modulo m, as int8.

    The result r satisfies r = X (mod m) and -floor(m/2) <= r <= ceil(m/2) - 1
    (Ozaki II notes §6: residues lie in [-128, 127]).  ``np.fmod`` of two
    doubles is exact, so no rounding enters.
    """
    r = np.fmod(np.asarray(X, dtype=np.float64), float(m))   # in (-m, m), sign of X
    r = np.where(r < 0, r + m, r)                              # in [0, m)
    r = np.where(r >= (m + 1) // 2, r - m, r)                  # in [-floor(m/2), ceil(m/2)-1]
    return r.astype(np.int8)


def residue_product(At: np.ndarray, Bt: np.ndarray) -> np.ndarray:
    """C'_t = A'_t B'_t for int8 residue matrices, exact, as int64
    (Ozaki II notes §4).

    Every product is an integer of magnitude <= 2^14 and every partial sum of
    a length-q dot product is an integer of magnitude <= q 2^14, inside the
    53-bit float64 significand for q < 2^39, so a float64 matrix product is
    exact in any summation order.  (§6: below q = 2^17 these values also fit
    int32; for larger q the notes split K into blocks, which changes nothing
    in the value of C'_t mod m_t, the only thing the method uses.)
    """
    q = At.shape[1]
    if q >= 2**39:
        raise ValueError("q >= 2^39: float64 partial sums would not be exact")
    C = np.asarray(At, dtype=np.float64) @ np.asarray(Bt, dtype=np.float64)
    return C.astype(np.int64)


def reduce_product(Ct: np.ndarray, m: int) -> np.ndarray:
    """C''_t = C'_t mod m_t, non-negative representative, as uint8
    (Ozaki II notes §4, §7 step 3)."""
    return np.mod(np.asarray(Ct, dtype=np.int64), m).astype(np.uint8)


# ----------------------------------------------------------------------------
# Steps 4-5: CRT accumulation and range reduction
# ----------------------------------------------------------------------------

def crt_combine(r: list[np.ndarray], moduli: list[int]) -> np.ndarray:
    """Z = sum_t C''_t M_t y_t, C''' = Z mod M, symmetric representative
    (Ozaki II notes §4 for the CRT sum, §5 for the range reduction).

    Returns an object array of Python ints X with |X| < M/2.  With 2 c_max < M
    the tie X = M/2 cannot occur; it is asserted absent.
    """
    M, Mt, yt = crt_constants(moduli)
    Z = np.zeros(np.asarray(r[0]).shape, dtype=object)
    for rt, Mt_t, yt_t in zip(r, Mt, yt):
        Z = Z + np.asarray(rt, dtype=np.int64).astype(object) * (Mt_t * yt_t)
    X = Z % M
    half = M // 2
    if M % 2 == 0:
        assert not np.any(X == half), "symmetric representative is ambiguous"
    X = np.where(X > half, X - M, X)
    return X


# ----------------------------------------------------------------------------
# Step 6: unscaling with a single rounding
# ----------------------------------------------------------------------------

def round_scaled(X: int, p: int) -> float:
    """X * 2^p rounded once to the nearest float64 (ties to even).

    Python's int -> float conversion and its int / int true division are both
    correctly rounded, subnormal range included; overflow becomes +-Inf.
    """
    X = int(X)
    if X == 0:
        return 0.0
    try:
        if p >= 0:
            return float(X << p)
        return X / (1 << (-p))
    except OverflowError:
        return math.copysign(math.inf, X)


def unscale(X: np.ndarray, e: np.ndarray, f: np.ndarray, k: int) -> np.ndarray:
    """C = D^-1 C''' E^-1, i.e. C_ij = RN(X_ij * 2^(e_i + f_j - 2k))
    (Ozaki II notes §7 step 6).  NaN where e_i or f_j is ``NONFINITE``."""
    m, n = X.shape
    C = np.empty((m, n), dtype=np.float64)
    for i in range(m):
        ei = int(e[i])
        for j in range(n):
            fj = int(f[j])
            if ei == NONFINITE or fj == NONFINITE:
                C[i, j] = math.nan
            else:
                C[i, j] = round_scaled(X[i, j], ei + fj - 2 * k)
    return C


# ----------------------------------------------------------------------------
# The whole scheme
# ----------------------------------------------------------------------------

# ----------------------------------------------------------------------------
# OS II-fast bit budget (Ozaki II notes §9)
# ----------------------------------------------------------------------------

#: Entries are rounded up on a grid of 2^-NORM_GRID (relative to 2^e) when
#: bounding row norms, so squared norms are integers in units of 2^-2*NORM_GRID.
NORM_GRID = 20


def cs_budget(M: int) -> tuple[int, int]:
    """(kappa_A, kappa_B) with kappa_A + kappa_B = floor(log2(M/2 - 1)).

    §9 (OS II-fast) bounds c_max with Cauchy-Schwarz instead of §5's
    q 2^(k_A + k_B): |(A'B')_ij| <= ||A'_i|| ||B'_j||.  Scaling every row of A'
    to norm <= 2^kappa_A and every column of B' to norm <= 2^kappa_B keeps
    2 c_max < M, the §5 uniqueness condition.  The budget is split evenly.
    """
    K2 = (M // 2 - 1).bit_length() - 1
    return K2 // 2, K2 - K2 // 2


def row_norm_units(A: np.ndarray, e: np.ndarray) -> list[int]:
    """S_i = sum_l ceil(|a_il| 2^(NORM_GRID - e_i))^2, an integer upper bound of
    ||a_i 2^-e_i||^2 in units of 2^(-2 NORM_GRID).  0 for rows that are zero
    or hold Inf/NaN.  Each term is at most 2^(2 NORM_GRID) and q < 2^23, so the
    int64 sums are exact."""
    A = np.asarray(A, dtype=np.float64)
    assert A.shape[1] < 2**23
    out = []
    for i in range(A.shape[0]):
        if e[i] == NONFINITE:
            out.append(0)
            continue
        t = np.ceil(np.ldexp(np.abs(A[i, :]), NORM_GRID - int(e[i]))).astype(np.int64)  # exact, <= 2^NORM_GRID
        out.append(int(np.sum(t * t)))
    return out


def fast_exponents(A: np.ndarray, e: np.ndarray, kappa: int, kb: int) -> np.ndarray:
    """Exponents e'_i = kb - d_i for the OS II-fast scaling d_i = kappa - c_i - e_i,
    with 4^c_i the smallest power of four >= S_i 2^(-2 NORM_GRID).  Then
    ||trunc(a_i 2^d_i)|| <= 2^d_i ||a_i|| <= 2^kappa, and the kernels' shift
    kb - e'_i equals d_i.  Zero rows keep 0, non-finite rows NONFINITE."""
    S = row_norm_units(A, e)
    out = np.zeros(len(S), dtype=np.int64)
    for i, Si in enumerate(S):
        if e[i] == NONFINITE:
            out[i] = NONFINITE
        elif Si == 0:
            out[i] = 0
        else:
            b = (Si - 1).bit_length()          # ceil(log2 S_i)
            c = (b + 1) // 2 - NORM_GRID       # ceil(log2(S_i)/2) - NORM_GRID
            d = kappa - c - int(e[i])
            out[i] = kb - d
    return out


# ----------------------------------------------------------------------------
# OS II-accu bit budget (Ozaki II notes §9)
# ----------------------------------------------------------------------------
#
# §9: "accu" estimates the range c_max >= max_ij (|A'||B'|)_ij with an extra
# low-precision GEMM, so that k_A, k_B can be opened wider than a cheap bound
# allows.  Readings taken here (the page gives no more detail):
#
# * the low-precision GEMM is the method's own exact int8 product.  Every
#   x_il = |a_il| 2^-e_i in [0, 1) is rounded up into one of two int8 bands,
#   x <= H/127 + Lo/(127 * 128): H = ceil(127 x) for x >= 2^-7, Lo =
#   ceil(127 * 128 x) for 0 < x < 2^-7 (both in [1, 127]), zero otherwise.
#   Then sum_l x_il y_lj <= (HH + (HL + LH)/128 + LL/128^2) / 127^2, where HH
#   and HL + LH are int8 products (one of length q, one of length 2q) and
#   LL <= 127 min(sum_l Lo_il, sum_l Lo_lj).  Everything is an exact integer,
#   so the bound, and every decision taken from it, is reproducible;
# * the bound decides per-row and per-column bit counts a_i, b_j with
#   2^(a_i + b_j) N_ij / (127^2 2^14) <= M/2 - 1 for every (i, j), compared
#   exactly: T_ij = floor(log2((M/2 - 1) 127^2 2^14 / N_ij)) is the largest
#   integer sum a_i + b_j that entry allows, and with K2 = floor(log2(M/2 -
#   1)) the budget reads a_i + b_j + L_ij <= K2 for L_ij = K2 - T_ij (L_ij =
#   -inf for a zero bound).  First each column takes half of what its largest
#   L leaves, then each row the most its columns allow, then each column the
#   most its rows allow; both capped at ACCU_KMAX.  |A'_il| <= 2^a_i x_il, so
#   (|A'||B'|)_ij <= 2^(a_i + b_j) N_ij / (127^2 2^14) <= M/2 - 1: the CRT
#   result is the exact A'B' (§5);
# * the shift of row i is a_i - e_i; the exponents handed to the residue and
#   CRT steps are e'_i = ACCU_KMAX - a_i + e_i (shift base ACCU_KMAX), as for
#   OS II-fast.

#: Largest bit count of a row of A' or column of B' (|A'| < 2^76 < 2^78,
#: the widest integers the residue step reduces exactly).
ACCU_KMAX = 76

#: Band resolution: H, Lo in [0, 127]; the low band covers x < 2^-ACCU_BAND.
ACCU_RES = 127
ACCU_BAND = 7

#: L of a zero bound (no constraint on the row and column).
ACCU_LZERO = -128


def accu_bands(X: np.ndarray, e: np.ndarray):
    """(H, Lo) int64 arrays with |x_rl| <= H/127 + Lo/(127 2^7) for
    x_rl = |X_rl| 2^-e_r, rounded up exactly: x = M 2^-sh with the integer
    significand M of |X_rl|, and ceil(c M / 2^sh) is an integer ceiling.
    Rows with e_r = NONFINITE are zero."""
    X = np.abs(np.asarray(X, dtype=np.float64))
    e = np.asarray(e, dtype=np.int64)
    H = np.zeros(X.shape, dtype=np.int64)
    Lo = np.zeros(X.shape, dtype=np.int64)
    live = (X > 0) & (e[:, None] != NONFINITE)
    mant, ex = np.frexp(X[live])                     # X = mant 2^ex, mant in [0.5, 1)
    M = (mant * 2.0**53).astype(np.int64).astype(object)  # X = M 2^(ex - 53), exactly
    rows = np.nonzero(live)[0]
    sh = (53 + e[rows] - ex).astype(object)          # x = M 2^-sh, sh >= 1 since x < 1
    hi = (M << ACCU_BAND) >= (1 << sh)               # x >= 2^-7 (Python integers)
    c = np.where(hi, ACCU_RES, ACCU_RES << ACCU_BAND).astype(object)
    v = (-((-(c * M)) >> sh)).astype(np.int64)       # ceil(c x), an exact integer ceiling
    hi = hi.astype(bool)
    H[live] = np.where(hi, v, 0)
    Lo[live] = np.where(hi, 0, v)
    return H, Lo


def ceil_log2_ratio(N: int, D: int) -> int:
    """Smallest integer L with N <= D 2^L, for integers N, D > 0."""
    L = N.bit_length() - D.bit_length()
    if (D << L if L >= 0 else D) < (N if L >= 0 else N << -L):
        L += 1
    return L


#: The two-band bound is N_ij / ACCU_DEN.
ACCU_DEN = ACCU_RES * ACCU_RES << (2 * ACCU_BAND)


def accu_bound(A: np.ndarray, B: np.ndarray, e: np.ndarray, f: np.ndarray) -> np.ndarray:
    """Integers N_ij with sum_l x_il y_lj <= N_ij / ACCU_DEN: the two-band
    int8 bound, N = 2^14 HH + 2^7 (HL + LH) + 127 min(sum_l Lo_il, sum_l Lo_lj).
    The int8 products are exact in float64 (every partial sum is an integer
    below 3 q 127^2 < 2^53)."""
    Ha, La = accu_bands(A, e)
    Hb, Lb = accu_bands(np.asarray(B).T, f)
    assert A.shape[1] * 3 * ACCU_RES**2 < 2**53
    HH = (Ha.astype(np.float64) @ Hb.T.astype(np.float64)).astype(np.int64)
    X = (Ha.astype(np.float64) @ Lb.T.astype(np.float64) + La.astype(np.float64) @ Hb.T.astype(np.float64)
         ).astype(np.int64)
    RS, CS = La.sum(axis=1), Lb.sum(axis=1)
    return (HH << (2 * ACCU_BAND)) + (X << ACCU_BAND) + ACCU_RES * np.minimum(RS[:, None], CS[None, :])


def accu_bound_exponents(A: np.ndarray, B: np.ndarray, e: np.ndarray, f: np.ndarray) -> np.ndarray:
    """L_ij = ceil(log2(N_ij / ACCU_DEN)) of :func:`accu_bound`, so that
    2^L_ij >= sum_l x_il y_lj (ACCU_LZERO where the bound is 0)."""
    N = accu_bound(A, B, e, f)
    D = ACCU_DEN
    L = np.full(N.shape, ACCU_LZERO, dtype=np.int64)
    for (i, j) in zip(*np.nonzero(N)):
        L[i, j] = ceil_log2_ratio(int(N[i, j]), D)
    return L


def accu_budget_exponents(A: np.ndarray, B: np.ndarray, e: np.ndarray, f: np.ndarray, M: int) -> np.ndarray:
    """L_ij = K2 - T_ij with T_ij = floor(log2((M/2 - 1) ACCU_DEN / N_ij)),
    the largest integer t with 2^t N_ij / ACCU_DEN <= M/2 - 1, and K2 =
    floor(log2(M/2 - 1)) (ACCU_LZERO where N_ij = 0).  The budget
    a_i + b_j + L_ij <= K2 is then exactly 2^(a_i + b_j) N_ij / ACCU_DEN <=
    M/2 - 1.  Python integers throughout: floor(log2(V / N)) is the bit length
    of V // N, less one."""
    N = accu_bound(A, B, e, f)
    V = (M // 2 - 1) * ACCU_DEN
    K2 = (M // 2 - 1).bit_length() - 1
    L = np.full(N.shape, ACCU_LZERO, dtype=np.int64)
    for (i, j) in zip(*np.nonzero(N)):
        L[i, j] = K2 - ((V // int(N[i, j])).bit_length() - 1)
    return L


def accu_scaling(L: np.ndarray, K2: int):
    """Bit counts (a_i, b_j) from the exponents L_ij of the bound, with
    a_i + b_j + L_ij <= K2 everywhere: columns take half of what their
    largest L leaves, rows the most their columns then allow, columns the
    most their rows then allow; all capped at ACCU_KMAX."""
    L = np.asarray(L, dtype=np.int64)
    b = np.minimum((K2 - L.max(axis=0)) // 2, ACCU_KMAX)
    a = np.minimum((K2 - L - b[None, :]).min(axis=1), ACCU_KMAX)
    b = np.minimum((K2 - L - a[:, None]).min(axis=0), ACCU_KMAX)
    return a, b


def accu_exponents(A: np.ndarray, B: np.ndarray, M: int):
    """Exponents (e'_i, f'_j) of OS II-accu for the shift base ACCU_KMAX:
    e'_i = ACCU_KMAX - a_i + e_i (row shift a_i - e_i); NONFINITE kept."""
    e = row_exponents(A).astype(np.int64)
    f = col_exponents(B).astype(np.int64)
    K2 = (M // 2 - 1).bit_length() - 1
    L = accu_budget_exponents(A, B, e, f, M)
    a, b = accu_scaling(L, K2)
    ep = np.where(e == NONFINITE, NONFINITE, ACCU_KMAX - a + e)
    fp = np.where(f == NONFINITE, NONFINITE, ACCU_KMAX - b + f)
    return ep, fp


def dgemm(A: np.ndarray, B: np.ndarray, s: int, stages: bool = False, bound: str = "conservative"):
    """C ~= A B by Ozaki Scheme II with s moduli (Ozaki II notes §7).

    ``bound`` selects the bit budget: "conservative" is §5's
    c_max <= q 2^(k_A + k_B) with k_A = k_B = k; "fast" is the §9 OS II-fast
    Cauchy-Schwarz budget of :func:`cs_budget` and :func:`fast_exponents`;
    "accu" is the §9 OS II-accu budget of :func:`accu_exponents` (the row
    and column bit counts depend on the whole of A and B, so a block of the
    result is not the result of the block's rows and columns).

    With ``stages=True`` also returns a dict of every intermediate:
    ``moduli, M, k, e, f, Ap, Bp, Ares (s x m x q int8), Bres (s x q x n int8),
    Ct (s x m x n int32), rt (s x m x n uint8), X (object), C``.  In fast and
    accu mode ``k`` is the shift base and e, f are the exponents e' of
    :func:`fast_exponents` or :func:`accu_exponents` (row shift k - e'_i).
    """
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    m, q = A.shape
    q2, n = B.shape
    if q != q2:
        raise ValueError("inner dimensions differ")
    mods = greedy_moduli(s)
    M, _, _ = crt_constants(mods)
    if q == 0:
        C = np.zeros((m, n))
        return (C, {"moduli": mods, "M": M, "k": None, "C": C}) if stages else C
    e = row_exponents(A)
    f = col_exponents(B)
    if bound == "conservative":
        k = kbits(M, q)
        if k < 1:
            raise ValueError(f"s={s} leaves no bits for q={q}")
    elif bound == "fast":
        kA, kB = cs_budget(M)
        k = max(kA, kB)
        e = fast_exponents(A, e, kA, k)
        f = fast_exponents(B.T, f, kB, k)
    elif bound == "accu":
        if kbits(M, q) < 1:
            raise ValueError(f"s={s} leaves no bits for q={q}")
        k = ACCU_KMAX
        e, f = accu_exponents(A, B, M)
    else:
        raise ValueError(f"unknown bound {bound!r}")
    Ap = truncate_rows(A, e, k)
    Bp = truncate_cols(B, f, k)
    Ares, Bres, Ct, rt = [], [], [], []
    for mt in mods:
        At = smod(Ap, mt)
        Bt = smod(Bp, mt)
        Ct_t = residue_product(At, Bt)
        Ares.append(At)
        Bres.append(Bt)
        Ct.append(Ct_t)
        rt.append(reduce_product(Ct_t, mt))
    X = crt_combine(rt, mods)
    C = unscale(X, e, f, k)
    if not stages:
        return C
    return C, {
        "moduli": mods, "M": M, "k": k, "e": e, "f": f, "Ap": Ap, "Bp": Bp,
        "Ares": np.stack(Ares), "Bres": np.stack(Bres), "Ct": np.stack(Ct),
        "rt": np.stack(rt), "X": X, "C": C,
    }


def dgemm_block(A: np.ndarray, B: np.ndarray, s: int, rows, cols, stages: bool = False, bound: str = "conservative"):
    """The oracle on the sub-problem A[rows, :] x B[:, cols].

    Exponents depend only on their own row of A or column of B and k only on
    q (in fast mode the budget only on M), so these are exactly the entries
    (rows x cols) of ``dgemm(A, B, s)``.  Used to check sampled outputs of
    problems too large for the full oracle.
    """
    A = np.asarray(A)
    B = np.asarray(B)
    return dgemm(A[np.asarray(rows), :], B[:, np.asarray(cols)], s, stages=stages, bound=bound)


# ----------------------------------------------------------------------------
# Exact reference product (for correct-bit measurements and error bounds)
# ----------------------------------------------------------------------------

def _exact_int(x: float):
    """x = mant * 2^expo with integer mant (exact decomposition of a double)."""
    mant, expo = math.frexp(x)
    return int(mant * (1 << 53)), expo - 53


def exact_dot(a: np.ndarray, b: np.ndarray):
    """Exact sum_l a_l b_l of two float64 vectors as ``(N, p)`` meaning N * 2^p."""
    terms = []
    for x, y in zip(np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)):
        if x == 0.0 or y == 0.0:
            continue
        mx, ex = _exact_int(float(x))
        my, ey = _exact_int(float(y))
        terms.append((mx * my, ex + ey))
    if not terms:
        return 0, 0
    p = min(t[1] for t in terms)
    return sum(v << (ep - p) for v, ep in terms), p


def correct_bits(C: np.ndarray, A: np.ndarray, B: np.ndarray, rows, cols) -> float:
    """-log2 max |C_ij - (AB)_ij| / (|A||B|)_ij over the given entries, with
    (AB)_ij computed exactly.  Returns 64.0 for an exact match everywhere."""
    from fractions import Fraction
    worst = Fraction(0)
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    absB = np.abs(B)
    for i, j in zip(rows, cols):
        N, p = exact_dot(A[i, :], B[:, j])
        exact = Fraction(N) * (Fraction(2) ** p)
        Na, pa = exact_dot(np.abs(A[i, :]), absB[:, j])
        denom = Fraction(Na) * (Fraction(2) ** pa)
        if denom == 0:
            continue
        err = abs(Fraction(float(C[i, j])) - exact) / denom
        worst = max(worst, err)
    if worst == 0:
        return 64.0
    return -math.log2(float(worst))
