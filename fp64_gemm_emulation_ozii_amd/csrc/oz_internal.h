// Internal declarations shared by the host library and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "../../include/ozgemm.h"
#include "crt_reconstruct.h"
#include "gemm_grid.h"

namespace oz {

// Tiling constants.  Residue planes are padded so that every kernel works on
// whole tiles: rows to ROW_PAD, the inner dimension to K_PAD.
constexpr int ROW_PAD = 256;
constexpr int K_PAD = 128;
constexpr int MAX_LIMBS = 5;      // 32-bit limbs of M: log2 M < 160 for s <= 20
constexpr int SCALE_CHUNK = 128;  // columns of A per partial row-max block

inline size_t round_up(size_t x, size_t r) { return (x + r - 1) / r * r; }

// |x| as its IEEE bit pattern: for non-negative doubles the unsigned integer
// order is the numeric order, and Inf/NaN patterns sort above every finite
// value (the scale step and the column residue kernel take maxima on these).
__device__ __forceinline__ uint64_t abs_bits(double x) {
  return (uint64_t)__double_as_longlong(x) & 0x7fffffffffffffffull;
}

__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// frexp exponent of the double whose |.| bit pattern is b:
// 2^(e - 1) <= |x| < 2^e; 0 for zero, OZGEMM_EXP_NONFINITE for Inf/NaN.
__device__ __forceinline__ int32_t exponent_of_bits(uint64_t b) {
  if (b == 0) return 0;
  if (b >= 0x7ff0000000000000ull) return OZGEMM_EXP_NONFINITE;
  int biased = (int)(b >> 52);
  if (biased > 0) return biased - 1022;         // value in [2^(E-1023), 2^(E-1022))
  int top = 63 - __clzll((long long)b);          // subnormal: mant * 2^-1074
  return top - 1073;
}

// OS II-fast norm bound (Ozaki II notes §9, Cauchy-Schwarz): the squared
// norm of a row x (or column) scaled by 2^-e is bounded by the exact integer
// S = sum ceil(|x| 2^(NORM_GRID - e))^2 in units of 2^(-2 NORM_GRID); any
// summation order gives the same S.
constexpr int NORM_GRID = 20;

// ceil(|x| 2^(NORM_GRID - e))^2 as an exact integer (|x| < 2^e).
__device__ __forceinline__ uint64_t norm_term(double x, int e) {
  const double t = __builtin_ceil(__builtin_ldexp(__builtin_fabs(x), NORM_GRID - e));
  const uint64_t u = (uint64_t)t;
  return u * u;
}

// e'_i from e_i and the squared-norm bound S (units 2^-2 NORM_GRID): the
// row is scaled by 2^d, d = kappa - c - e with 4^c the smallest power of
// four >= S 2^(-2 NORM_GRID), and handed on as e' = kb - d.
__device__ __forceinline__ int32_t fast_exponent(int32_t e, uint64_t S, int kappa, int kb) {
  if (e == OZGEMM_EXP_NONFINITE) return e;
  if (S == 0) return 0;
  const int b = (S == 1) ? 0 : 64 - __clzll((long long)(S - 1));  // ceil(log2 S)
  const int c = (b + 1) / 2 - NORM_GRID;
  return kb - (kappa - c - e);
}

// Per-modulus constants for the residue kernel (Ozaki II notes §6).
struct ResidueConsts {
  int s;
  int k;                        // shift base: row shift is k - e_i
  int kmag;                     // |A'| < 2^kmag (selects the residue arithmetic)
  int col_kappa;                // B in one pass under OS II-fast: kappa_B (-1: the exponent as it is)
  int m[OZGEMM_S_MAX];          // moduli
  double inv[OZGEMM_S_MAX];     // RN(1/m)
  double c26[OZGEMM_S_MAX];     // 2^26 mod m
  double c52[OZGEMM_S_MAX];     // 2^52 mod m
};

// Per-modulus constants for the GEMM epilogue.
struct GemmConsts {
  int s;
  int m[OZGEMM_S_MAX];
  double inv[OZGEMM_S_MAX];
};

// CRT constants (Ozaki II notes §4).  The W-bit limbs of W_t = M_t y_t < M
// are stored as doubles in a device table (wtab[t * MAX_LIMBS + l]) so that
// sum_t r_t W_t accumulates exactly in FP64; the rest travels by value.
struct CrtConsts {
  int s;
  int W;                             // limb width: 40 (log2 M <= 120) or 32
  int L;                             // limbs of M (top limb nonzero)
  int k;
  const double* wtab;                // device: s x MAX_LIMBS limbs of W_t
  CrtModulus K;                      // limbs of M and M/2, M/2, 1/M
};

// Host table of the W_t limbs for every s (wtab for s at (s - 1) * S_MAX * MAX_LIMBS).
constexpr size_t CRT_TABLE_DOUBLES = (size_t)OZGEMM_S_MAX * OZGEMM_S_MAX * MAX_LIMBS;

// Launchers (each enqueues on `st`).
hipError_t launch_row_max_partial(const double* A, int m, int q, int lda, uint64_t* pmax, int m_stride,
                                  int nchunks, hipStream_t st);
hipError_t launch_row_exp_finalize(const uint64_t* pmax, int m, int m_stride, int nchunks, int32_t* e,
                                   hipStream_t st);
hipError_t launch_col_exp(const double* B, int q, int n, int ldb, int32_t* f, hipStream_t st);
// launch_row_max_partial and launch_col_exp as one launch (q >= 1).
hipError_t launch_scale_pair(const double* A, int m, int q, int lda, uint64_t* pmax, int m_stride, int nchunks,
                             const double* B, int n, int ldb, int32_t* f, hipStream_t st);
// OS II-fast: replace e (f) by e' (f') from Cauchy-Schwarz row (column) norm bounds.
hipError_t launch_row_fast(const double* A, int m, int q, int lda, uint64_t* psum, int m_stride, int nchunks,
                           int kappa, int kb, int32_t* e, hipStream_t st);
hipError_t launch_col_fast(const double* B, int q, int n, int ldb, int kappa, int kb, int32_t* f, hipStream_t st);
// launch_row_fast and launch_col_fast with A's and B's norm passes as one launch.
hipError_t launch_fast_pair(const double* A, int m, int q, int lda, uint64_t* psum, int m_stride, int nchunks,
                            int kappa_a, const double* B, int n, int ldb, int kappa_b, int kb, int32_t* e,
                            int32_t* f, hipStream_t st);

// Residues of the rows of X where element (r, l) sits at X[r*rs + l*ls].
// Writes `rows_pad` x q_pad int8 planes (plane stride rows_pad*q_pad).
// B's column exponents and residue planes in one pass (conservative bit
// budget, OZGEMM_ONE_PASS_Q_MIN <= q <= OZGEMM_ONE_PASS_Q_MAX); writes
// ex[0..rows) like launch_col_exp would.
bool col_residue_fits(int q);
hipError_t launch_col_residue(const double* X, int rows, int q, long rs, int32_t* ex, const ResidueConsts& c,
                              int8_t* planes, int rows_pad, int q_pad, hipStream_t st);
// The residues of column-major A (m x q) and B (q x n) as one launch, the
// same planes as two launch_residue calls write (m, n, q >= 1).  With pmax
// non-null, A's row exponents are not read from e but taken from the
// nchunks partial row maxima of the scale step (pmax[c * m_stride + i]) and
// written to e by the tiles of the first K columns: the row-exponent
// finalisation folded into this launch.
hipError_t launch_residue_pair(const double* A, int m, int lda, int32_t* e, int8_t* Aplanes, int m_pad,
                               const double* B, int n, int ldb, const int32_t* f, int8_t* Bplanes, int n_pad, int q,
                               int q_pad, const ResidueConsts& c, hipStream_t st, const uint64_t* pmax = nullptr,
                               int m_stride = 0, int nchunks = 0);
hipError_t launch_residue(const double* X, int rows, int q, long rs, long ls, const int32_t* ex,
                          const ResidueConsts& c, int8_t* planes, int rows_pad, int q_pad,
                          double* prime, long prime_rs, long prime_ls, hipStream_t st);

// Scheme II products C_t = A_t B_t^T: int32 planes Ct and/or residues mod m_t
// in rt.  With split.parts > 1 (residue-only) the K parts write the planes
// `parts` (split.parts * s planes of m_pad * n_pad bytes; may be rt itself)
// and are summed into rt; see gemm_grid.h.  Residue-only products with more
// blocks than cus (the device's compute units; 0 = never) run as cus
// persistent blocks that walk the tiles.
hipError_t launch_gemm(const int8_t* Ares, const int8_t* Bres, int m_pad, int n_pad, int q_pad,
                       const GemmConsts& c, int32_t* Ct, uint8_t* rt, const SplitChoice& split, uint8_t* parts,
                       int cus, hipStream_t st);

// Scheme I slice products: output plane plan[o].w (m_pad x n_pad int32, [j][i])
// = sum over u < plan[o].z of A_{plan[o].x + u} B_{plan[o].y - u}^T.
hipError_t launch_gemm_multi(const int8_t* Aplanes, const int8_t* Bplanes, int m_pad, int n_pad, int q_pad,
                             const int4* plan, int nout, int32_t* P, hipStream_t st);

// Scheme I split and accumulation (scheme1.hip).
hipError_t launch_s1_rowmax(const double* X, int rows, int q, long rs, long ls, int rows_pad, int q_pad,
                            uint64_t* pmax, hipStream_t st);
hipError_t launch_s1_grid(const uint64_t* pmax, int rows_pad, int nchunks, int beta, int32_t* gout, hipStream_t st);
// Scheme I split of rows held in LDS (rows contiguous in memory, as the rows
// of B are), one pass for all k slices; same grids and slices as
// launch_s1_rowmax + launch_s1_grid + launch_s1_split.
bool s1_row_split_fits(int q);
hipError_t launch_s1_row_split(const double* X, int rows, int q, long rs, int rows_pad, int q_pad, int variant, int k,
                               int beta, int32_t* g, int8_t* planes, hipStream_t st);
hipError_t launch_s1_split(const double* X, int rows, int q, long rs, long ls, const int32_t* g, int rows_pad,
                           int q_pad, int variant, int pass, int k, int beta, int8_t* planes, uint64_t* pmax,
                           hipStream_t st);
hipError_t launch_s1_plan(int variant, int k, int r, int beta, int4* gemm_plan, int4* acc_plan, hipStream_t st);
hipError_t launch_s1_accum(const int32_t* P, int m, int n, int m_pad, int n_pad, int nout, const int4* acc,
                           const int32_t* gA, int ma_pad, const int32_t* gB, int nb_pad, double* C, int ldc,
                           hipStream_t st);

hipError_t launch_crt(const uint8_t* rt, int m, int n, int m_pad, int n_pad, const int32_t* e,
                      const int32_t* f, const CrtConsts& c, double* C, int ldc, hipStream_t st);

hipError_t launch_fill_zero(double* C, int m, int n, int ldc, hipStream_t st);

// OS II-accu (accu.hip): replace the row and column exponents e, f (frexp
// exponents of the maxima) by the exponents e', f' of the accu bit budget
// (shift base kmax, K2 = floor(log2(M/2 - 1)); V = (M/2 - 1) 127^2 2^14 has
// bv bits, the top 64 of them in vtop, see accu_budget_consts).  Aplanes / Bplanes
// hold 2 m_pad q_pad / 2 n_pad q_pad bytes of band planes, psumA
// 4 m_pad q_pad / 128 bytes, scratch accu_scratch_bytes(...) bytes; q_pad <= 2^16.
constexpr int ACCU_KMAX = 76;         // |A'| < 2^76: the residue step's widest exact integers
constexpr int ACCU_Q_MAX = 1 << 16;   // 2 127^2 q_pad < 2^31: the bound products are exact in int32
size_t accu_scratch_bytes(int m_pad, int n_pad, int q_pad);
hipError_t launch_accu_exponents(const double* A, int m, int q, int lda, const double* B, int n, int ldb, int m_pad,
                                 int n_pad, int q_pad, int K2, uint64_t vtop, int bv, int kmax, int8_t* Aplanes,
                                 int8_t* Bplanes, int32_t* psumA, char* scratch, int32_t* e, int32_t* f,
                                 hipStream_t st);

// Measurement aid (probe.hip): `blocks` workgroups of four wavefronts run
// `steps` register-only steps of 32 v_mfma_i32_16x16x64_i8 each; sink
// receives 4 blocks words.
hipError_t launch_mfma_ceiling(int blocks, int steps, uint32_t seed, uint32_t* sink, hipStream_t st);

}  // namespace oz
