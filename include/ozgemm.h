/*
 * ozgemm -- FP64 matrix multiplication C = A B emulated with exact
 * INT8 x INT8 -> INT32 matrix products (Ozaki Scheme II), for AMD MI355X
 * (gfx950).
 *
 * Method: the web page "Ozaki Scheme II：用 CRT 把高精度 GEMM 映射成少量 INT8
 * GEMM" (chatdocs.ruinique.com/nla/ozaki-scheme-ii), cited below as
 * "Ozaki II notes §n".  Its §7 lists the pipeline this library runs:
 *   1. bit budget k from M = prod m_t and the inner dimension q (§5);
 *   2. power-of-two row/column scalings D, E and truncation to integer
 *      matrices A' = trunc(DA), B' = trunc(BE) (§3);
 *   3. for each of s pairwise-coprime moduli m_t <= 256: symmetric int8
 *      residues of A' and B', one exact int8 GEMM, product mod m_t (§4, §6);
 *   4-5. CRT accumulation and reduction to the symmetric representative (§4, §5);
 *   6. unscaling by D^-1 and E^-1 (§7).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Matrices are column-major (BLAS convention): A is m x q with leading
 *    dimension lda >= max(1, m); B is q x n, ldb >= max(1, q); C is m x n,
 *    ldc >= max(1, m).  No alpha/beta: C is overwritten.  A caller holding
 *    row-major data passes (B^T, A^T) and receives C^T.
 *  - Every pointer argument that names matrix data is DEVICE memory owned by
 *    the caller; the library never allocates, frees or retains it.
 *  - Work is enqueued on the configured HIP stream and the calls return
 *    without synchronising (like BLAS on a GPU).  The caller synchronises.
 *  - Return value: 0 on success.  -i means argument i (1-based) is invalid;
 *    positive values are the OZGEMM_* codes below.  Arguments are checked
 *    before anything is enqueued, so outputs are untouched on any error.
 *  - The library keeps one global configuration; it is not thread-safe and
 *    calls that overlap on one stream-set race on the workspace.
 *  - s, the number of moduli, is 1..OZGEMM_S_MAX; the moduli are the first s
 *    of the greedy pairwise-coprime sequence 256, 255, 253, 251, 247, 241,
 *    239, 233, 229, 227, 223, 217, 211, 199, 197, 193, 191, 181, 179, 173.
 *  - Every int8 dot product of length < 2^17 (|.| <= q * 2^14) is exact in
 *    int32 (Ozaki II notes §6).  For q >= 2^17 the GEMM splits K into parts
 *    of at most 2^16 and adds their products mod m_t (the notes' block
 *    products; see ozgemm_gemm_parts), so q may go up to OZGEMM_Q_MAX; s
 *    must leave k >= 1 bits (§5).  Otherwise OZGEMM_RANGE.
 *  - Numerics: the result equals X * 2^(e_i + f_j - 2k) rounded once to
 *    nearest-even, where X = (A'B')_ij exactly.  Rows of A / columns of B that
 *    hold Inf or NaN make the outputs they touch NaN; all-zero rows/columns
 *    give +0; results beyond the double range round to +-Inf.
 */
#ifndef OZGEMM_H
#define OZGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define OZGEMM_OK                  0
#define OZGEMM_NOT_CONFIGURED      1  /* ozgemm_config has not succeeded */
#define OZGEMM_RANGE               2  /* q > OZGEMM_Q_MAX, k(s, q) < 1 (conservative budget), q >= OZGEMM_FAST_Q_LIMIT (OS II-fast), or size beyond the configured maximum */
#define OZGEMM_WORKSPACE_TOO_SMALL 3  /* workspace_bytes below ozgemm_workspace_bytes(...) */
#define OZGEMM_HIP_ERROR           4  /* a HIP call failed; ozgemm_strerror(4) names it */

#define OZGEMM_S_MAX 20               /* largest supported number of moduli */
#define OZGEMM_Q_LIMIT (1 << 17)      /* int8 dot products of length < this are exact in int32 (Ozaki II notes §6) */
#define OZGEMM_Q_MAX   (1 << 27)      /* largest supported inner dimension */
#define OZGEMM_FAST_Q_LIMIT (1 << 23) /* OS II-fast needs q below this: its row-norm sums of q terms of at most 2^40 stay exact in 64 bits */
#define OZGEMM_MAX_ROWS 2096896       /* largest m and n: 2^21 - 256, so that the rows padded to 256 form at most 65535 tiles of 32 */
#define OZGEMM_EXP_NONFINITE 0x7fffffff /* exponent of a row/column holding Inf/NaN */
#define OZGEMM_PANELS_MAX 16          /* most column panels of the pipeline (ozgemm_set_panels) */
#define OZGEMM_ONE_PASS_Q_MIN 4096    /* ozgemm_dgemm reads B once for Q_MIN <= q <= Q_MAX (conservative budget) */
#define OZGEMM_ONE_PASS_Q_MAX 8192

/* Bit budgets of Scheme II (ozgemm_set_bound) */
#define OZGEMM_BOUND_CONSERVATIVE 0 /* c_max <= q 2^(k_A + k_B), k_A = k_B = k (Ozaki II notes §5) */
#define OZGEMM_BOUND_FAST         1 /* Cauchy-Schwarz c_max bound, OS II-fast (Ozaki II notes §9) */
#define OZGEMM_BOUND_ACCU         2 /* c_max bound from an extra exact int8 product, OS II-accu (Ozaki II notes §9) */
#define OZGEMM_ACCU_Q_MAX   (1 << 16) /* OS II-accu needs q <= this: its bound products stay exact in int32 */

/* Scheme I variants (Ozaki I notes, optimized algorithm) */
#define OZGEMM_S1_RN      0  /* RN split, per-product FP64 accumulation (direction 1) */
#define OZGEMM_S1_HYBRID  1  /* Hybrid split, group-wise INT32 accumulation (directions 2, 3) */
#define OZGEMM_S1_K_MAX   16 /* largest number of slices */
#define OZGEMM_S1_MAX_OUT 136 /* k (k + 1) / 2 at k = OZGEMM_S1_K_MAX */

/* ---------------------------------------------------------------------- */
/* Configuration                                                          */
/* ---------------------------------------------------------------------- */

/* Bytes of device workspace needed for problems up to max_m x max_n x max_q
 * with up to s_max moduli (the per-modulus int8 residue planes of A and B,
 * the uint8 product residues -- at least 128 MiB of them when max_q >= 3969,
 * for the K parts of skinny products -- and small per-row/column arrays).
 * Returns 0 for invalid arguments.  Host only. */
size_t ozgemm_workspace_bytes(int max_m, int max_n, int max_q, int s_max);

/* Record the maximum problem size, the HIP stream (a hipStream_t, may be
 * NULL for the null stream) and a caller-owned device workspace of
 * workspace_bytes bytes.  Nothing is allocated or launched.  Replaces any
 * previous configuration.  Errors: -1..-4 bad sizes (max_m and max_n at most
 * OZGEMM_MAX_ROWS, max_q at most OZGEMM_Q_MAX), -6 NULL workspace,
 * OZGEMM_WORKSPACE_TOO_SMALL. */
int ozgemm_config(int s_max, int max_m, int max_n, int max_q,
                  void *hip_stream, void *workspace, size_t workspace_bytes);

/* Change the stream used by later calls. */
int ozgemm_set_stream(void *hip_stream);

/* Column-panel pipeline of ozgemm_dgemm (Ozaki II notes §8 and §11: the
 * CRT of one part of C overlaps the products of the next part).  C is cut
 * into P column panels of whole 256-column tiles; each panel's B residues
 * and product residues are contiguous, its product is one launch, and its
 * CRT runs on a second stream of the library (default priority, created at
 * the first pipelined call and released by ozgemm_free or ozgemm_config),
 * ordered by events, while the next panel's product runs.  The call's
 * stream waits for the last CRT, so the call stays one unit of work on that
 * stream (and can be captured into a graph like an unpipelined one).
 * Results are identical to the unpipelined path.
 *   panels = 0 or 1: no pipeline (the default);
 *   2 <= panels <= OZGEMM_PANELS_MAX: that many panels whenever the shape
 *     allows (q < 2^17, n_pad >= 512, one K part per panel product).
 * It is off by default because on MI355X the persistent product grid holds
 * every compute unit, so the CRT only fills gaps: measured 1.5-2% slower
 * than the plain call at 16384 x 16384 x 1024 and 8192^3.
 * The setting persists until changed; ozgemm_free resets it to 0.
 * Returns 0, or -1 for panels outside 0..OZGEMM_PANELS_MAX. */
int ozgemm_set_panels(int panels);

/* Forget the configuration (the workspace stays the caller's). */
int ozgemm_free(void);

/* Text for a status code; for OZGEMM_HIP_ERROR it includes the HIP error. */
const char *ozgemm_strerror(int status);

/* ---------------------------------------------------------------------- */
/* The hot path                                                           */
/* ---------------------------------------------------------------------- */

/* C <- A B by Ozaki Scheme II with s moduli (Ozaki II notes §7).
 * m, n, q >= 0; m = 0 or n = 0 does nothing; q = 0 writes C = 0.
 * C must not overlap A or B (-8).  Requires m <= max_m, n <= max_n,
 * q <= max_q, s <= s_max of the configuration (OZGEMM_RANGE otherwise).
 * Enqueues the scale, residue, int8 GEMM and CRT kernels on the stream.
 * Under the conservative budget with OZGEMM_ONE_PASS_Q_MIN <= q <=
 * OZGEMM_ONE_PASS_Q_MAX, B's column exponents are taken inside its residue
 * pass, so B is read once; A is read twice (its row maxima need every column
 * first).  Shorter columns keep two passes, whose first is cheap there.  The
 * results are the same as those of the stage entry points.
 * The first call after ozgemm_config also copies a 16 KB constant table
 * into the workspace (a blocking host-to-device copy) and queries the
 * device's compute-unit count; later calls only enqueue kernels, so they can
 * be captured into a HIP graph once one call has run outside capture. */
int ozgemm_dgemm(int m, int n, int q,
                 const double *A, int lda, const double *B, int ldb,
                 double *C, int ldc, int s);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): C <- A B
 * exactly as ozgemm_dgemm computes it (same kernels, same bit budget as set
 * by ozgemm_set_bound, same results), with every intermediate in a fixed
 * device array of OZGEMM_NOALLOC_BYTES bytes that the library holds on each
 * GPU it runs on until the process ends.  Needs no ozgemm_config; work goes
 * on `hip_stream` (a hipStream_t, NULL for the null stream) and the call
 * returns without synchronising.  The caller passes device pointers A, B, C
 * as for ozgemm_dgemm.  Calls no hipMalloc, hipFree or other allocating
 * routine.  The first call on a device looks up the array's address and
 * copies a 16 KB constant table into it (a blocking host-to-device copy), so
 * make one call outside any graph capture first.
 * The array is shared by every call on that GPU and keeps the last call's
 * contents: calls that overlap on one GPU (other streams, other host
 * threads) race on it and give wrong results.  Products are not cut into K
 * parts here (q >= 2^17 walks sequential K blocks).
 * Errors: those of ozgemm_dgemm (argument numbers 1..10; no
 * OZGEMM_NOT_CONFIGURED), and OZGEMM_RANGE when the intermediates of this
 * shape need more than OZGEMM_NOALLOC_BYTES: s (m_pad + n_pad) q_pad bytes of
 * residue planes, s m_pad n_pad of product residues (under OS II-accu at
 * least the bound's planes, about 9.02 m_pad n_pad bytes), 2 KB per padded
 * row of A for partial row maxima, and small arrays (m_pad, n_pad: m, n
 * rounded up to 256; q_pad: q rounded up to 128).  ozgemm_workspace_bytes(m, n, q, s)
 * <= OZGEMM_NOALLOC_BYTES is enough; for example 2048 x 2048 x 1024 fits at
 * s = 14, and 1024^3 at every s. */
#define OZGEMM_NOALLOC_BYTES (128 << 20)
int ozgemm_dgemm_noalloc(int m, int n, int q,
                         const double *A, int lda, const double *B, int ldb,
                         double *C, int ldc, int s, void *hip_stream);

/* ---------------------------------------------------------------------- */
/* Host-only introspection (no device needed)                              */
/* ---------------------------------------------------------------------- */

/* Write the first s moduli to moduli_out[0..s-1].  Returns 0 or -1. */
int ozgemm_moduli(int s, int *moduli_out);

/* k = floor(1/2 log2((M/2 - 1)/q)) for the first s moduli, evaluated with
 * exact integers (Ozaki II notes §5), for 1 <= q <= OZGEMM_Q_MAX (long inner
 * dimensions run as K parts, see ozgemm_gemm_parts).  Returns k, which is
 * < 1 when s and q leave no bits (ozgemm_dgemm then returns OZGEMM_RANGE
 * under the conservative budget); -1 for s outside 1..OZGEMM_S_MAX or q < 1;
 * -2 for q > OZGEMM_Q_MAX. */
int ozgemm_kbits(int s, int q);

/* Padded dimensions of the stage buffers below: rows of the residue planes
 * are padded to *m_pad / *n_pad, the inner dimension to *q_pad. */
int ozgemm_plane_dims(int m, int n, int q, int *m_pad, int *n_pad, int *q_pad);

/* Bit budget of later Scheme II calls (ozgemm_dgemm and its stages); the
 * setting persists until changed (ozgemm_free resets it to conservative).
 *   OZGEMM_BOUND_CONSERVATIVE: k = floor(1/2 log2((M/2 - 1)/q)) bits per
 *     entry of every row of A and column of B (Ozaki II notes §5).
 *   OZGEMM_BOUND_FAST: OS II-fast (Ozaki II notes §9).  With
 *     kappa_A + kappa_B = floor(log2(M/2 - 1)) split evenly, row i of A is
 *     scaled by 2^d_i, d_i = kappa_A - c_i - e_i, where 4^c_i is the smallest
 *     power of four >= S_i 2^-40 and S_i = sum_l ceil(|a_il| 2^(20 - e_i))^2
 *     (an exact integer bound of ||a_i 2^-e_i||^2 in units of 2^-40); columns
 *     of B likewise with kappa_B.  Then ||A'_i|| ||B'_j|| <= 2^(kappa_A +
 *     kappa_B) < M/2 (Cauchy-Schwarz), so the CRT result is still the exact
 *     A'B', and entries keep more bits whenever a row's norm is well below
 *     sqrt(q) times its maximum.  The stage exponents become
 *     e'_i = kb - d_i with kb = max(kappa_A, kappa_B), so that the row shift
 *     is kb - e'_i and the unscaling exponent e'_i + f'_j - 2 kb.  Needs
 *     q < OZGEMM_FAST_Q_LIMIT.
 *   OZGEMM_BOUND_ACCU: OS II-accu (Ozaki II notes §9): c_max is bounded by
 *     an extra exact int8 product.  With x_il = |a_il| 2^-e_i in [0, 1)
 *     (e_i the frexp exponent of the row maximum; y_lj likewise for the
 *     columns of B), each x is rounded up into two int8 bands,
 *     x <= H/127 + Lo/(127 2^7): H = ceil(127 x) for x >= 2^-7, Lo =
 *     ceil(127 2^7 x) below.  Then sum_l x_il y_lj <= N_ij / (127^2 2^14)
 *     with N = 2^14 H_A H_B^T + 2^7 (H_A Lo_B^T + Lo_A H_B^T) +
 *     127 min(row sum of Lo_A, column sum of Lo_B), two int8 products run
 *     on the product kernel (length q and 2q).  Row bit counts a_i and
 *     column bit counts b_j satisfy 2^(a_i + b_j) N_ij / (127^2 2^14) <=
 *     M/2 - 1 for every (i, j), compared exactly (a_i + b_j + L_ij <= K2
 *     with K2 = floor(log2(M/2 - 1)) and L_ij = K2 - floor(log2((M/2 - 1)
 *     127^2 2^14 / N_ij))): columns first take half of what their largest
 *     L leaves, rows then the most their columns allow, columns then the
 *     most their rows allow, all at most 76.  Row i of A' is
 *     trunc(a_il 2^(a_i - e_i)), so (|A'||B'|)_ij < M/2 and the CRT result
 *     is exact (§5).  The stage exponents are
 *     e'_i = 76 - a_i + e_i (shift base 76).  Every quantity is an exact
 *     integer, so results are reproducible.  Needs q <= OZGEMM_ACCU_Q_MAX,
 *     s >= 2 and k(s, q) >= 1, and room in the workspace's product region
 *     for two int32 planes and one int8 plane of m_pad x n_pad (about 9.02
 *     m_pad n_pad bytes, which s_max >= 10 always gives; otherwise
 *     OZGEMM_WORKSPACE_TOO_SMALL).
 * Returns 0, or -1 for an unknown mode. */
int ozgemm_set_bound(int mode);

/* Bit budget for (s, q) under `mode`: (k, k) for the conservative bound
 * (OZGEMM_RANGE if k < 1), (kappa_A, kappa_B) for OS II-fast (OZGEMM_RANGE
 * if q >= OZGEMM_FAST_Q_LIMIT), (K2, 76) for OS II-accu: the budget
 * a_i + b_j + L_ij <= K2 = floor(log2(M/2 - 1)) that the row and column bit
 * counts share, and their cap (OZGEMM_RANGE if q > OZGEMM_ACCU_Q_MAX, s < 2
 * or k < 1). */
int ozgemm_bound_budget(int s, int q, int mode, int *kappa_a, int *kappa_b);

/* ---------------------------------------------------------------------- */
/* Stage entry points (the same kernels ozgemm_dgemm runs), for parity     */
/* checks of each integer stage.  All buffers are caller-owned device      */
/* memory; the configured workspace and stream are used.                   */
/* ---------------------------------------------------------------------- */

/* Exponents (Ozaki II notes §3, §5): e[i] for i < m with
 * 2^(e_i - 1) <= max_l |a_il| < 2^e_i (0 for an all-zero row,
 * OZGEMM_EXP_NONFINITE for a row holding Inf/NaN); f[j] likewise for the
 * columns of B.  e has m entries, f has n.  Under OZGEMM_BOUND_FAST the
 * values are the shift exponents e'_i, f'_j of that budget (see
 * ozgemm_set_bound), which depend on s. */
int ozgemm_stage_scale(int m, int n, int q, int s,
                       const double *A, int lda, const double *B, int ldb,
                       int32_t *e, int32_t *f);

/* Truncation and residues (Ozaki II notes §3, §4, §6), with k = kbits(s, q):
 *   A'_il = trunc(a_il 2^(k - e_i)),  B'_lj = trunc(b_lj 2^(k - f_j)),
 *   Ares[t][i][l] = smod(A'_il, m_t),  Bres[t][j][l] = smod(B'_lj, m_t),
 * smod(x, m) in [-floor(m/2), ceil(m/2) - 1].  Planes are int8, K-contiguous:
 * Ares at t*m_pad*q_pad + i*q_pad + l, Bres at t*n_pad*q_pad + j*q_pad + l,
 * zero in the padding.  Aprime (m x q, ld m) and Bprime (q x n, ld q) are
 * optional (NULL to skip) float64 copies of A' and B'. */
int ozgemm_stage_residue(int m, int n, int q, int s,
                         const double *A, int lda, const double *B, int ldb,
                         const int32_t *e, const int32_t *f,
                         int8_t *Ares, int8_t *Bres,
                         double *Aprime, double *Bprime);

/* Per-modulus products (Ozaki II notes §4, §6): C_t = A_t B_t^T over q_pad,
 * exact in int32.  Ct (optional, NULL to skip) receives int32 planes,
 * column-major with ld m_pad: Ct[t*m_pad*n_pad + j*m_pad + i].  rt
 * (optional) receives C_t mod m_t in [0, m_t) as uint8 in the same layout.
 * Without Ct, the product may run as K parts (ozgemm_gemm_parts) whose
 * planes use the workspace's product region; rt must not lie in the
 * workspace. */
int ozgemm_stage_gemm(int m, int n, int q, int s,
                      const int8_t *Ares, const int8_t *Bres,
                      int32_t *Ct, uint8_t *rt);

/* Number of K parts the residue-only product of an m x n x q call with s
 * moduli runs as (ozgemm_dgemm, and ozgemm_stage_gemm without Ct), written
 * to *parts.  When moduli x output tiles of 256 x 256 leave the compute
 * units idle, the inner dimension is cut into P parts, one block per (part,
 * modulus, tile); each part's product mod m_t goes to a plane of the
 * workspace, and a reduction adds the P residues mod m_t (the sum of the
 * parts is the whole product; a part of at most 2^16 K entries is exact in
 * int32, Ozaki II notes §6).  1 = one part; 0 = q >= 2^17 with no room for
 * parts, walked as sequential K blocks instead.  The choice depends on the
 * device's compute units (queried on the current device) and on the
 * configured workspace.  Errors: -1..-5, OZGEMM_NOT_CONFIGURED,
 * OZGEMM_RANGE, OZGEMM_HIP_ERROR. */
int ozgemm_gemm_parts(int m, int n, int q, int s, int *parts);

/* CRT reconstruction, range reduction and unscaling (Ozaki II notes §4, §5,
 * §7): from rt (layout of ozgemm_stage_gemm), e and f, write the m x n result
 * C (ld ldc). */
int ozgemm_stage_crt(int m, int n, int q, int s,
                     const uint8_t *rt, const int32_t *e, const int32_t *f,
                     double *C, int ldc);

/* ---------------------------------------------------------------------- */
/* Scheme I: FP64 GEMM from int8 slices (secondary path)                   */
/*                                                                        */
/* Method: the course page "Ozaki Scheme" (zsc0tt.pages.dev/courses/      */
/* hpc-summer/ozaki-scheme), cited as "Ozaki I notes": its optimized      */
/* algorithm after Uchino, Ozaki and Imamura.  Each row of A and column  */
/* of B is split into k signed slices of beta bits,                       */
/* beta = min(7, floor((31 - log2 q) / 2)); slice p of a row is the       */
/* row's remaining residual rounded to nearest-even on a power-of-two     */
/* grid 2^g (|slice / 2^g| <= 2^(beta-1)).  The products A_i B_j with     */
/* i + j <= k + 1 (k (k + 1) / 2 of them) are exact int8 GEMMs and are    */
/* added up in FP64 in a fixed order, so results are reproducible.        */
/*   OZGEMM_S1_RN:     grid of slice p from the max of the row's residual */
/*                     (RN split); each product converted and added,      */
/*                     i-major, j-minor.                                  */
/*   OZGEMM_S1_HYBRID: grid of slice p = g0 - beta (p - 1), g0 from the   */
/*                     original row max (Hybrid split); products with the */
/*                     same i + j summed in int32, at most                */
/*                     r = max(1, 2^(31 - 2 beta - ceil(log2 q))) at a    */
/*                     time, then added in increasing i + j.              */
/* Grid exponents: g = ceil(log2 max|row|) + 1 - beta; 0 for an all-zero  */
/* row; OZGEMM_EXP_NONFINITE (first grid row only) for a row holding      */
/* Inf/NaN, whose slices are zero and whose outputs are NaN.              */
/* These calls use the configured stream and workspace; the workspace     */
/* must hold ozgemm_scheme1_workspace_bytes(m, n, q, k, variant) bytes    */
/* (else OZGEMM_WORKSPACE_TOO_SMALL).  q may exceed 2^17 (beta shrinks);  */
/* beta < 1 (q > 2^29) gives OZGEMM_RANGE.                                */
/* ---------------------------------------------------------------------- */

/* Slice width beta for inner dimension q, or -1 when none fits. */
int ozgemm_scheme1_beta(int q);

/* Number of int32 product planes (outputs of the products stage):
 * k (k + 1) / 2 for RN; the number of runs for Hybrid.  <0 on bad input. */
int ozgemm_scheme1_outputs(int k, int variant, int q);

/* Workspace bytes needed by a Scheme I call of this shape (0 on bad input). */
size_t ozgemm_scheme1_workspace_bytes(int m, int n, int q, int k, int variant);

/* C <- A B by Scheme I with k slices (1 <= k <= OZGEMM_S1_K_MAX).
 * Arguments and conventions as ozgemm_dgemm, with k and variant in place
 * of s.  Phase timing slots: [scale: 0, split, products, accumulation]. */
int ozgemm_scheme1_dgemm(int m, int n, int q,
                         const double *A, int lda, const double *B, int ldb,
                         double *C, int ldc, int k, int variant);

/* Split stage (Ozaki I notes, RN split / Hybrid split algorithms).
 * Aslices[p][i][l] (p < k) at p*m_pad*q_pad + i*q_pad + l: slice integers of
 * row i of A; Bslices[p][j][l] at p*n_pad*q_pad + j*q_pad + l for column j of
 * B (int8, zero in the padding; m_pad, n_pad, q_pad from ozgemm_plane_dims).
 * gA[p][i] at p*m_pad + i and gB[p][j] at p*n_pad + j: grid exponents, k
 * rows for RN, one row (g0) for Hybrid. */
int ozgemm_scheme1_stage_split(int m, int n, int q, int k, int variant,
                               const double *A, int lda, const double *B, int ldb,
                               int8_t *Aslices, int8_t *Bslices,
                               int32_t *gA, int32_t *gB);

/* Products stage: P[o][j][i] at o*m_pad*n_pad + j*m_pad + i (int32) for
 * o < ozgemm_scheme1_outputs(k, variant, q), in accumulation order:
 * RN: o-th pair (i, j) of the triangle, P = A_i B_j^T;
 * Hybrid: o-th run of pairs (s, g - s), P = sum of their products. */
int ozgemm_scheme1_stage_products(int m, int n, int q, int k, int variant,
                                  const int8_t *Aslices, const int8_t *Bslices,
                                  int32_t *P);

/* Accumulation stage: C (m x n, ld ldc) = sum over o, in order, of
 * P[o] scaled by 2^(gA + gB) of its slices (Hybrid: 2^(g0A + g0B - beta (g - 2))),
 * each addition rounded in FP64. */
int ozgemm_scheme1_stage_accumulate(int m, int n, int q, int k, int variant,
                                    const int32_t *P, const int32_t *gA,
                                    const int32_t *gB, double *C, int ldc);

/* ---------------------------------------------------------------------- */
/* Phase timing                                                           */
/* ---------------------------------------------------------------------- */

/* enable != 0: every later ozgemm_dgemm records HIP events on the stream
 * around its four phases (up to 4096 calls).  ozgemm_phase_ms adds, over the
 * calls since timing was enabled, the milliseconds of [scale, residue, gemm,
 * crt] into ms_out[0..3] (synchronising on the events) and the number of
 * calls into *calls (for a pipelined call, see ozgemm_set_panels: residue =
 * A's residues, gemm = B's residues, the products and the overlapped CRTs,
 * crt = the last panel's CRT tail).  ozgemm_phase_calls writes the same four times of each
 * call, ms_out[4c + p] for call c < min(calls, max_calls), and the number of
 * recorded calls into *calls (either pointer may be NULL when max_calls is
 * 0).  Disabling discards the events. */
int ozgemm_timing(int enable);
int ozgemm_phase_ms(double *ms_out, int *calls);
int ozgemm_phase_calls(double *ms_out, int max_calls, int *calls);

/* Measurement aid: the rate the int8 matrix cores sustain on their own, the
 * practical ceiling of the product step (Ozaki II notes §6: one int8 GEMM
 * per modulus; §10 reports the method against the int8 rate).  `blocks`
 * workgroups of four wavefronts each run `steps` steps of 32
 * v_mfma_i32_16x16x64_i8 with operands in registers, in the product
 * kernel's issue order (2^20 int8 operations per wavefront and step), on
 * pseudo-random operands from `seed`.  Each wavefront writes the XOR of its
 * accumulator words to sink[4 * block + wavefront] (device memory,
 * 4 * blocks uint32, caller owned), which makes the result checkable.
 * Asynchronous on hip_stream (NULL: the null stream); time it with events
 * on that stream.  Needs no configuration.  Returns 0, -1 for blocks
 * outside 1..2^20, -2 for steps < 1, -4 for sink == NULL, or
 * OZGEMM_HIP_ERROR. */
int ozgemm_mfma_ceiling(int blocks, int steps, unsigned seed, unsigned *sink, void *hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* OZGEMM_H */
