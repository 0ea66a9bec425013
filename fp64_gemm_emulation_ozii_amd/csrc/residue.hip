// Residue step: truncation to integers and symmetric int8 residues, fused.
//
// Ozaki II notes §3: A' = trunc(DA) with D = diag(2^(k - e_i)); §4: one
// residue matrix per modulus; §6: moduli <= 256 with symmetric residues in
// [-floor(m/2), ceil(m/2) - 1], which fit signed int8; §15 asks for scaling,
// truncation, modulo and int8 packing in one kernel, which this is.
//
// Each block converts a tile of TR rows x TK inner-dimension entries.  The
// doubles are staged through LDS so that the global reads are coalesced
// whatever the source layout (rows contiguous for column-major A, the inner
// dimension contiguous for column-major B), and every thread then owns 16
// consecutive inner-dimension entries of one row and writes them as one
// 16-byte store per modulus into the K-contiguous plane the GEMM reads.
//
// Exactness.  a * 2^(k - e) is exact (a power-of-two scaling) unless it
// falls below 2^-1022, where it is below 1 and truncates to 0 anyway.  The
// residues of the truncated integers come from residue_arith.h: one
// uncorrected reduction per modulus while |A'| < 2^50, and for wider A'
// (|A'| < 2^78 since k <= 77 for s <= 20) a split into 26-bit pieces once per
// entry, then 5 or 6 FP64 operations per modulus, where a +-m correction
// (50 < k <= 53) or a second reduction of a 2^32 high part (k > 53) took 8
// (same calls at 8192^3: 2.5% faster at s = 15 under the conservative
// budget, 0.7-0.9% under OS II-fast at s = 14 and 15).
#include "oz_internal.h"
#include "residue_arith.h"

namespace oz {

namespace {

constexpr int TR = 32;           // rows per tile
constexpr int TK = 128;          // inner-dimension entries per tile
constexpr int LDS_STRIDE = TK + 1;  // doubles; odd stride spreads banks

// Low bytes of four words as one word (three byte permutes).
__device__ __forceinline__ uint32_t pack_bytes(uint32_t b0, uint32_t b1, uint32_t b2, uint32_t b3) {
  const uint32_t lo = __builtin_amdgcn_perm(b1, b0, 0x0c0c0400u);  // b0.0, b1.0, 0, 0
  const uint32_t hi = __builtin_amdgcn_perm(b3, b2, 0x0c0c0400u);  // b2.0, b3.0, 0, 0
  return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

// The s residues of 16 consecutive entries of one row, A' exact integers in
// a[] (|A'| < 2^kmag), as one 16-byte store per modulus at dst + t plane_stride.
template <int MODE>  // 0: kmag <= 50, 1: kmag <= 53, 2: kmag > 53
__device__ __forceinline__ void write_residues16(double (&a)[16], const ResidueConsts& c, int8_t* dst,
                                                 long plane_stride) {
  if (MODE == 0) {  // |A'| < 2^50 (residue_arith.h)
    double am[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) am[j] = a[j] + 0x1.8p52;
    for (int t = 0; t < c.s; ++t) {
      const double md = (double)c.m[t], inv = c.inv[t];
      uint32_t rb[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) rb[j] = residue_narrow(a[j], am[j], md, inv);
      uint4 out;
      out.x = pack_bytes(rb[0], rb[1], rb[2], rb[3]);
      out.y = pack_bytes(rb[4], rb[5], rb[6], rb[7]);
      out.z = pack_bytes(rb[8], rb[9], rb[10], rb[11]);
      out.w = pack_bytes(rb[12], rb[13], rb[14], rb[15]);
      *reinterpret_cast<uint4*>(dst + (long)t * plane_stride) = out;
    }
    return;
  }
  // |A'| >= 2^50: split once into 26-bit pieces, one reduction per modulus
  // (residue_arith.h)
  constexpr bool BIG = MODE == 2;
  double a1[16], a2[16] = {};
#pragma unroll
  for (int j = 0; j < 16; ++j) split_wide<BIG>(a[j], a1[j], a2[j]);
  for (int t = 0; t < c.s; ++t) {
    const double md = (double)c.m[t], inv = c.inv[t], c26 = c.c26[t];
    const double c52 = BIG ? c.c52[t] : 0.0;
    uint32_t rb[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) rb[j] = (uint32_t)residue_wide<BIG>(a[j], a1[j], a2[j], c26, c52, md, inv);
    uint4 out;
    out.x = pack_bytes(rb[0], rb[1], rb[2], rb[3]);
    out.y = pack_bytes(rb[4], rb[5], rb[6], rb[7]);
    out.z = pack_bytes(rb[8], rb[9], rb[10], rb[11]);
    out.w = pack_bytes(rb[12], rb[13], rb[14], rb[15]);
    *reinterpret_cast<uint4*>(dst + (long)t * plane_stride) = out;
  }
}

// The row-exponent finalisation folded into A's residue tiles: the partial
// row maxima of the scale step (nchunks words per row, stride m_stride) and
// where the exponents go.
struct FoldedExp {
  const uint64_t* pmax;
  int m_stride;
  int nchunks;
  int32_t* e_out;
};

// Tile (bx, by) of residue_kernel: rows by*TR.., inner-dimension entries
// bx*TK.., staged through `tile` (TR * LDS_STRIDE doubles of LDS).  With
// FOLD the row exponents come from the partial row maxima (the eight threads
// of a row each take every eighth chunk) instead of ex, and the tiles with
// bx = 0 write them to fold.e_out.
template <bool ROWS_CONTIG, int MODE, bool FOLD = false>  // MODE 0: k <= 50, 1: k <= 53, 2: k > 53
__device__ __forceinline__ void residue_tile(double* tile, int bx, int by, const double* __restrict__ X, int rows,
                                             int q, long rs, long ls, const int32_t* __restrict__ ex,
                                             const ResidueConsts& c, int8_t* __restrict__ planes, long plane_stride,
                                             int q_pad, double* __restrict__ prime, long prime_rs, long prime_ls,
                                             FoldedExp fold = {nullptr, 0, 0, nullptr}) {
  const int tid = threadIdx.x;
  const int r0 = by * TR;
  const int l0 = bx * TK;
  const int grow = r0 + (tid >> 3);  // the row this thread converts (below)

  // partial maxima first, so that their latency overlaps the tile's loads
  uint64_t pm = 0;
  if (FOLD && grow < rows)
    for (int cc = tid & 7; cc < fold.nchunks; cc += 8) pm = umax64(pm, fold.pmax[(long)cc * fold.m_stride + grow]);

  // ---- coalesced load into LDS (zero outside the matrix) ----
  // All loads are issued before any is used: out-of-range lanes read a
  // clamped, valid element and store zero instead (q >= 1; with no rows at
  // all nothing is read and the tile is zero padding).
  if (rows < 1) {
    for (int idx = tid; idx < TR * LDS_STRIDE; idx += 256) tile[idx] = 0.0;
  } else if (ROWS_CONTIG) {
    // consecutive lanes -> consecutive rows of one column
    const int r = tid & (TR - 1);
    const int lsub = tid >> 5;  // 0..7
    const bool rok = (r0 + r) < rows;
    const double* src = X + (long)min(r0 + r, rows - 1);
    double v[TK / 8];
#pragma unroll
    for (int it = 0; it < TK / 8; ++it)
      v[it] = __builtin_nontemporal_load(src + (long)min(l0 + lsub + 8 * it, q - 1) * ls);
#pragma unroll
    for (int it = 0; it < TK / 8; ++it) {
      const int l = lsub + 8 * it;
      tile[r * LDS_STRIDE + l] = (rok && (l0 + l) < q) ? v[it] : 0.0;
    }
  } else {
    // consecutive lanes -> consecutive inner-dimension entries of one row
    const int l = tid & (TK - 1);
    const int rsub = tid >> 7;  // 0..1
    const bool lok = (l0 + l) < q;
    const double* src = X + (long)min(l0 + l, q - 1);
    double v[TR / 2];
#pragma unroll
    for (int it = 0; it < TR / 2; ++it)
      v[it] = __builtin_nontemporal_load(src + (long)min(r0 + rsub + 2 * it, rows - 1) * rs);
#pragma unroll
    for (int it = 0; it < TR / 2; ++it) {
      const int r = rsub + 2 * it;
      tile[r * LDS_STRIDE + l] = (lok && (r0 + r) < rows) ? v[it] : 0.0;
    }
  }
  __syncthreads();

  // ---- each thread: one row, 16 consecutive entries ----
  const int r = tid >> 3;          // 0..31
  const int cseg = (tid & 7) * 16; // 0..112
  int e = 0;
  bool zero_row = true;
  if (FOLD) {
    // the row's maximum over the eight threads of the row (lanes 8 j .. 8 j + 7)
#pragma unroll
    for (int off = 1; off < 8; off <<= 1) pm = umax64(pm, (uint64_t)__shfl_xor((unsigned long long)pm, off, 64));
    if (grow < rows) {
      e = exponent_of_bits(pm);
      zero_row = (e == OZGEMM_EXP_NONFINITE);
      if (bx == 0 && (tid & 7) == 0) fold.e_out[grow] = e;
    }
  } else if (grow < rows) {
    e = ex[grow];
    zero_row = (e == OZGEMM_EXP_NONFINITE);
  }
  const int shift = zero_row ? 0 : c.k - e;

  double a[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    double x = tile[r * LDS_STRIDE + cseg + j];
    double t = __builtin_trunc(__builtin_ldexp(x, shift));
    a[j] = zero_row ? 0.0 : t + 0.0;  // + 0.0 turns -0.0 into +0.0
  }

  if (prime != nullptr && grow < rows) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int gl = l0 + cseg + j;
      if (gl < q) prime[(long)grow * prime_rs + (long)gl * prime_ls] = a[j];
    }
  }

  write_residues16<MODE>(a, c, planes + (long)grow * q_pad + l0 + cseg, plane_stride);
}

template <bool ROWS_CONTIG, int MODE>
__global__ __launch_bounds__(256) void residue_kernel(const double* __restrict__ X, int rows, int q, long rs,
                                                       long ls, const int32_t* __restrict__ ex, ResidueConsts c,
                                                       int8_t* __restrict__ planes, long plane_stride, int q_pad,
                                                       double* __restrict__ prime, long prime_rs, long prime_ls) {
  __shared__ double tile[TR * LDS_STRIDE];
  residue_tile<ROWS_CONTIG, MODE>(tile, blockIdx.x, blockIdx.y, X, rows, q, rs, ls, ex, c, planes, plane_stride,
                                  q_pad, prime, prime_rs, prime_ls);
}

// A's and B's residues in one launch (column-major A: rows contiguous; B:
// the inner dimension contiguous): blocks [0, na) are A's tiles, the rest
// B's, each in row-major order of a (q_pad / TK)-wide grid.  For small
// products the two passes' ramp-up and drain then overlap.
template <int MODE, bool FOLD>
__global__ __launch_bounds__(256) void residue_pair_kernel(const double* __restrict__ A, int m, long lda,
                                                            const int32_t* __restrict__ e,
                                                            int8_t* __restrict__ Aplanes, int m_pad,
                                                            const double* __restrict__ B, int n, long ldb,
                                                            const int32_t* __restrict__ f,
                                                            int8_t* __restrict__ Bplanes, int n_pad, int q, int q_pad,
                                                            ResidueConsts c, int na, FoldedExp fold) {
  __shared__ double tile[TR * LDS_STRIDE];
  const int gx = q_pad / TK;
  const int b = blockIdx.x;
  if (b < na)
    residue_tile<true, MODE, FOLD>(tile, b % gx, b / gx, A, m, q, 1, lda, e, c, Aplanes, (long)m_pad * q_pad,
                                   q_pad, nullptr, 0, 0, fold);
  else
    residue_tile<false, MODE>(tile, (b - na) % gx, (b - na) / gx, B, n, q, ldb, 1, f, c, Bplanes,
                              (long)n_pad * q_pad, q_pad, nullptr, 0, 0);
}

// B in one pass (Ozaki II notes §15: scaling, truncation, modulo and packing
// fused): one block per row j of the B planes, i.e. per column of B, which
// is contiguous.  The block loads the column into LDS (coalesced, all loads
// in flight before any is used), takes the frexp exponent of its largest
// |b_lj| (written to ex[j], exactly as the scale step computes it), and then
// converts it like residue_kernel: each thread owns 16 consecutive entries
// and writes one 16-byte store per modulus.  One pad double after every 16
// makes those 16-entry reads conflict-free (64 lanes touch 32 distinct
// 8-byte bank pairs twice).  Rows j >= rows and entries l >= q are padding
// and get zero residues.
constexpr int COL_QMAX = OZGEMM_ONE_PASS_Q_MAX;  // longest column held
constexpr int COL_LDS = COL_QMAX + COL_QMAX / 16;  // doubles, with the pads

template <int MODE>
__global__ __launch_bounds__(256) void col_residue_kernel(const double* __restrict__ X, int rows, int q, long rs,
                                                           int32_t* __restrict__ ex, ResidueConsts c,
                                                           int8_t* __restrict__ planes, long plane_stride,
                                                           int q_pad) {
  __shared__ double col[COL_LDS];
  __shared__ uint64_t wmax[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j = blockIdx.x;
  int e = 0;
  bool zero_row = true;
  if (j < rows) {  // uniform across the block
    const double* src = X + (long)j * rs;
    double v[COL_QMAX / 256];
#pragma unroll
    for (int i = 0; i < COL_QMAX / 256; ++i) {
      const int l = tid + 256 * i;
      v[i] = l < q ? __builtin_nontemporal_load(src + l) : 0.0;
    }
    uint64_t mx = 0;
#pragma unroll
    for (int i = 0; i < COL_QMAX / 256; ++i) {
      const int l = tid + 256 * i;
      mx = umax64(mx, abs_bits(v[i]));
      col[l + (l >> 4)] = v[i];
    }
    for (int off = 32; off > 0; off >>= 1) mx = umax64(mx, (uint64_t)__shfl_xor((unsigned long long)mx, off, 64));
    if (lane == 0) wmax[wave] = mx;
    __syncthreads();
    e = exponent_of_bits(umax64(umax64(wmax[0], wmax[1]), umax64(wmax[2], wmax[3])));
    zero_row = (e == OZGEMM_EXP_NONFINITE);
    if (c.col_kappa >= 0) {  // uniform: OS II-fast, the column's norm bound from the same registers
      uint64_t S = 0;
      if (!zero_row) {
#pragma unroll
        for (int i = 0; i < COL_QMAX / 256; ++i) S += norm_term(v[i], e);  // zero past q
      }
      for (int off = 32; off > 0; off >>= 1) S += (uint64_t)__shfl_xor((unsigned long long)S, off, 64);
      __syncthreads();  // every wave has read wmax
      if (lane == 0) wmax[wave] = S;
      __syncthreads();
      e = fast_exponent(e, wmax[0] + wmax[1] + wmax[2] + wmax[3], c.col_kappa, c.k);
    }
    if (tid == 0) ex[j] = e;
  }
  __syncthreads();
  const int shift = zero_row ? 0 : c.k - e;
  for (int seg = tid; seg < q_pad / 16; seg += 256) {
    double a[16];
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
      const double x = col[17 * seg + jj];  // entry 16 seg + jj, past its pads
      const double t = __builtin_trunc(__builtin_ldexp(x, shift));
      a[jj] = zero_row ? 0.0 : t + 0.0;  // + 0.0 turns -0.0 into +0.0
    }
    write_residues16<MODE>(a, c, planes + (long)j * q_pad + 16 * seg, plane_stride);
  }
}
}  // namespace

hipError_t launch_residue(const double* X, int rows, int q, long rs, long ls, const int32_t* ex,
                          const ResidueConsts& c, int8_t* planes, int rows_pad, int q_pad, double* prime,
                          long prime_rs, long prime_ls, hipStream_t st) {
  if (q < 1) return hipErrorInvalidValue;  // q = 0 has no residues (callers handle it)
  if (q_pad % TK || rows_pad % TR || q_pad < q || rows_pad < rows) return hipErrorInvalidValue;  // whole tiles
  if (rows_pad / TR > 65535) return hipErrorInvalidValue;  // grid.y
  dim3 grid(q_pad / TK, rows_pad / TR);
  const long plane_stride = (long)rows_pad * q_pad;
  const bool rows_contig = (rs == 1);
  const int mode = c.kmag <= 50 ? 0 : (c.kmag <= 53 ? 1 : 2);
#define OZ_RES_LAUNCH(RC, MD)                                                                                \
  hipLaunchKernelGGL((residue_kernel<RC, MD>), grid, dim3(256), 0, st, X, rows, q, rs, ls, ex, c, planes,     \
                     plane_stride, q_pad, prime, prime_rs, prime_ls)
  if (rows_contig) {
    if (mode == 0) OZ_RES_LAUNCH(true, 0);
    else if (mode == 1) OZ_RES_LAUNCH(true, 1);
    else OZ_RES_LAUNCH(true, 2);
  } else {
    if (mode == 0) OZ_RES_LAUNCH(false, 0);
    else if (mode == 1) OZ_RES_LAUNCH(false, 1);
    else OZ_RES_LAUNCH(false, 2);
  }
#undef OZ_RES_LAUNCH
  return hipGetLastError();
}

hipError_t launch_residue_pair(const double* A, int m, int lda, int32_t* e, int8_t* Aplanes, int m_pad,
                               const double* B, int n, int ldb, const int32_t* f, int8_t* Bplanes, int n_pad, int q,
                               int q_pad, const ResidueConsts& c, hipStream_t st, const uint64_t* pmax,
                               int m_stride, int nchunks) {
  if (q < 1 || m < 1 || n < 1) return hipErrorInvalidValue;
  if (q_pad % TK || m_pad % TR || n_pad % TR || q_pad < q || m_pad < m || n_pad < n)
    return hipErrorInvalidValue;  // whole tiles
  if (pmax != nullptr && (nchunks < 1 || m_stride < m)) return hipErrorInvalidValue;
  const long na = (long)(q_pad / TK) * (m_pad / TR), nb = (long)(q_pad / TK) * (n_pad / TR);
  if (na + nb > 0x7fffffffL) return hipErrorInvalidValue;
  const int mode = c.kmag <= 50 ? 0 : (c.kmag <= 53 ? 1 : 2);
  const FoldedExp fold{pmax, m_stride, nchunks, e};
#define OZ_RES_PAIR(MD, FD)                                                                                    \
  hipLaunchKernelGGL((residue_pair_kernel<MD, FD>), dim3((unsigned)(na + nb)), dim3(256), 0, st, A, m, (long)lda, \
                     FD ? nullptr : e, Aplanes, m_pad, B, n, (long)ldb, f, Bplanes, n_pad, q, q_pad, c, (int)na,  \
                     fold)
  if (pmax != nullptr) {
    if (mode == 0) OZ_RES_PAIR(0, true);
    else if (mode == 1) OZ_RES_PAIR(1, true);
    else OZ_RES_PAIR(2, true);
  } else {
    if (mode == 0) OZ_RES_PAIR(0, false);
    else if (mode == 1) OZ_RES_PAIR(1, false);
    else OZ_RES_PAIR(2, false);
  }
#undef OZ_RES_PAIR
  return hipGetLastError();
}

// Shorter columns keep the two-pass path: a block per column of under 4096
// entries is too little work for its 68 KB of LDS, and the separate scale
// read of such a B is cheap (measured at 16384^2 x 1024: the one-pass B took
// 0.29 ms against 0.14 + 0.02 ms for the two passes).
bool col_residue_fits(int q) { return q >= OZGEMM_ONE_PASS_Q_MIN && q <= COL_QMAX; }

hipError_t launch_col_residue(const double* X, int rows, int q, long rs, int32_t* ex, const ResidueConsts& c,
                              int8_t* planes, int rows_pad, int q_pad, hipStream_t st) {
  if (!col_residue_fits(q) || q_pad > COL_QMAX || q_pad % 16 || rows_pad < rows) return hipErrorInvalidValue;
  const long plane_stride = (long)rows_pad * q_pad;
  const int mode = c.kmag <= 50 ? 0 : (c.kmag <= 53 ? 1 : 2);
#define OZ_COL_LAUNCH(MD)                                                                                    \
  hipLaunchKernelGGL((col_residue_kernel<MD>), dim3(rows_pad), dim3(256), 0, st, X, rows, q, rs, ex, c, planes, \
                     plane_stride, q_pad)
  if (mode == 0) OZ_COL_LAUNCH(0);
  else if (mode == 1) OZ_COL_LAUNCH(1);
  else OZ_COL_LAUNCH(2);
#undef OZ_COL_LAUNCH
  return hipGetLastError();
}

}  // namespace oz
