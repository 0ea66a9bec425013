// OS II-accu bit budget (Ozaki II notes §9): a range estimate of c_max from
// an extra low-precision product, which lets every row of A and column of B
// keep as many bits as the CRT range allows.
//
// Bound.  With x_il = |a_il| 2^-e_i and y_lj = |b_lj| 2^-f_j in [0, 1) (e, f
// the frexp exponents of the row and column maxima), every x is rounded up
// into one of two int8 bands: H = ceil(127 x) for x >= 2^-7, Lo =
// ceil(127 2^7 x) for 0 < x < 2^-7, both in [1, 127]; so x <= H/127 +
// Lo/(127 2^7).  Then
//   sum_l x_il y_lj <= N_ij / (127^2 2^14),
//   N_ij = 2^14 HH_ij + 2^7 (HL + LH)_ij + 127 min(RS_i, CS_j),
// where HH = H_A H_B^T and HL + LH = H_A Lo_B^T + Lo_A H_B^T are exact int8
// products on the matrix cores (the plan form of the product kernel: one of
// length q, one of length 2q; exact in int32 while 2 127^2 q_pad < 2^31) and
// RS_i, CS_j are the row sums of Lo (LL = Lo_A Lo_B^T <= 127 min(RS_i, CS_j)).
//
// Budget.  Entry (i, j) admits a_i + b_j <= T_ij = floor(log2(V / N_ij)),
// V = (M/2 - 1) 127^2 2^14, the largest t with 2^t N_ij / (127^2 2^14) <=
// M/2 - 1, compared exactly; it is kept as L_ij = K2 - T_ij with K2 =
// floor(log2(M/2 - 1)), or -128 (no constraint) for N = 0.
//
// Scaling.  Bit counts a_i, b_j with a_i + b_j + L_ij <= K2 for all (i, j),
// so that (|A'||B'|)_ij <= 2^(a_i + b_j) N_ij / (127^2 2^14) < M/2 and the CRT
// result is exact (§5): each column first takes half of what its largest L
// leaves, each row then the most its columns allow, each column then the most
// its rows allow; all at most ACCU_KMAX.  The exponents handed on are e'_i = ACCU_KMAX - a_i + e_i (row
// shift a_i - e_i, shift base ACCU_KMAX), NONFINITE kept.
//
// Every quantity is an exact integer function of the inputs, so the result
// does not depend on the order of any sum.
#include "oz_internal.h"
#include "accu_budget.h"

namespace oz {

namespace {

constexpr int TR = 32;              // rows per band tile
constexpr int TK = 128;             // inner-dimension entries per band tile
constexpr int LDS_STRIDE = TK + 1;  // doubles; odd stride spreads banks
constexpr int RES = 127;            // band resolution
constexpr double LOW_EDGE = 0x1p-7; // x below this goes to the low band
constexpr int LZERO = -128;         // L of a zero bound
constexpr int CHUNK = 256;          // columns per block of the row-minimum pass

// ceil(c x) for 0 <= x < 1 and c = 127 or 127 * 128, exactly: p = RN(c x)
// and the product's rounding error err = c x - p (exact by fma).  If p is an
// integer, c x exceeds it exactly when err > 0; otherwise no integer lies
// between p and c x (rounding is monotone and integers are doubles).
__device__ __forceinline__ int ceil_mul(double c, double x) {
  const double p = c * x;
  const double err = __builtin_fma(c, x, -p);
  const double cp = __builtin_ceil(p);
  return (int)cp + ((cp == p && err > 0.0) ? 1 : 0);
}

__device__ __forceinline__ uint32_t pack4(const int* v) {
  return (uint32_t)(v[0] & 0xff) | ((uint32_t)(v[1] & 0xff) << 8) | ((uint32_t)(v[2] & 0xff) << 16) |
         ((uint32_t)(v[3] & 0xff) << 24);
}

// Tile (bx, by) of the bands of the rows of X (element (r, l) at
// X[r rs + l ls]) into two int8 planes (rows_pad x q_pad, K-contiguous, zero
// padding), and per tile of 128 inner-dimension entries the sum of each
// row's Lo values: psum[bx * rows_pad + r].  `tile` is TR * LDS_STRIDE
// doubles of LDS.
template <bool ROWS_CONTIG>
__device__ __forceinline__ void band_tile(double* tile, int bx, int by, const double* __restrict__ X, int rows, int q,
                                          long rs, long ls, const int32_t* __restrict__ ex, int8_t* __restrict__ Hp,
                                          int8_t* __restrict__ Lp, int q_pad, int rows_pad,
                                          int32_t* __restrict__ psum) {
  const int tid = threadIdx.x;
  const int r0 = by * TR;
  const int l0 = bx * TK;
  if (rows < 1) {
    for (int idx = tid; idx < TR * LDS_STRIDE; idx += 256) tile[idx] = 0.0;
  } else if (ROWS_CONTIG) {
    const int r = tid & (TR - 1);
    const int lsub = tid >> 5;
    const bool rok = (r0 + r) < rows;
    const double* src = X + (long)min(r0 + r, rows - 1);
    double v[TK / 8];
#pragma unroll
    for (int it = 0; it < TK / 8; ++it) v[it] = src[(long)min(l0 + lsub + 8 * it, q - 1) * ls];
#pragma unroll
    for (int it = 0; it < TK / 8; ++it) {
      const int l = lsub + 8 * it;
      tile[r * LDS_STRIDE + l] = (rok && (l0 + l) < q) ? v[it] : 0.0;
    }
  } else {
    const int l = tid & (TK - 1);
    const int rsub = tid >> 7;
    const bool lok = (l0 + l) < q;
    const double* src = X + (long)min(l0 + l, q - 1);
    double v[TR / 2];
#pragma unroll
    for (int it = 0; it < TR / 2; ++it) v[it] = src[(long)min(r0 + rsub + 2 * it, rows - 1) * rs];
#pragma unroll
    for (int it = 0; it < TR / 2; ++it) {
      const int r = rsub + 2 * it;
      tile[r * LDS_STRIDE + l] = (lok && (r0 + r) < rows) ? v[it] : 0.0;
    }
  }
  __syncthreads();

  const int r = tid >> 3;            // 0..31
  const int cseg = (tid & 7) * 16;   // 0..112
  const int grow = r0 + r;           // < rows_pad
  int e = 0;
  bool live = false;
  if (grow < rows) {
    e = ex[grow];
    live = e != OZGEMM_EXP_NONFINITE;
  }
  int h[16], lo[16];
  int sum = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const double a = __builtin_fabs(tile[r * LDS_STRIDE + cseg + j]);
    const double x = __builtin_ldexp(a, -e);  // exact unless below 2^-1022 (then in the low band)
    const bool nz = live && a != 0.0;
    const bool hi = x >= LOW_EDGE;
    const int hv = ceil_mul((double)RES, x);
    const int lv = max(ceil_mul((double)(RES << 7), x), 1);  // a != 0 lost to underflow still counts 1
    h[j] = (nz && hi) ? hv : 0;
    lo[j] = (nz && !hi) ? lv : 0;
    sum += lo[j];
  }
  const long off = (long)grow * q_pad + l0 + cseg;
  *reinterpret_cast<uint4*>(Hp + off) = make_uint4(pack4(h), pack4(h + 4), pack4(h + 8), pack4(h + 12));
  *reinterpret_cast<uint4*>(Lp + off) = make_uint4(pack4(lo), pack4(lo + 4), pack4(lo + 8), pack4(lo + 12));
  // the 8 threads of a row are 8 consecutive lanes of one wavefront
#pragma unroll
  for (int o = 1; o < 8; o <<= 1) sum += __shfl_xor(sum, o, 64);
  if ((tid & 7) == 0) psum[(long)bx * rows_pad + grow] = sum;
}

// A's bands (column-major A: rows contiguous) and B's (its columns as rows:
// the inner dimension contiguous) in one launch: blocks [0, na) are A's
// tiles, the rest B's, each in row-major order of a (q_pad / TK)-wide grid.
__global__ __launch_bounds__(256) void accu_band_pair_kernel(
    const double* __restrict__ A, int m, long lda, const int32_t* __restrict__ e, int8_t* __restrict__ AH,
    int8_t* __restrict__ AL, int m_pad, int32_t* __restrict__ psumA, const double* __restrict__ B, int n, long ldb,
    const int32_t* __restrict__ f, int8_t* __restrict__ BH, int8_t* __restrict__ BL, int n_pad,
    int32_t* __restrict__ psumB, int q, int q_pad, int na) {
  __shared__ double tile[TR * LDS_STRIDE];
  const int gx = q_pad / TK;
  const int b = blockIdx.x;
  if (b < na)
    band_tile<true>(tile, b % gx, b / gx, A, m, q, 1L, lda, e, AH, AL, q_pad, m_pad, psumA);
  else
    band_tile<false>(tile, (b - na) % gx, (b - na) / gx, B, n, q, ldb, 1L, f, BH, BL, q_pad, n_pad, psumB);
}

// Row sums of Lo for A's rows (blocks [0, ga)) and B's columns (the rest):
// out[r] = sum over the nchunks tiles of psum, 64 rows per block, four
// threads per row each adding every fourth tile sum (eight loads in
// flight), combined through LDS.  (One thread per row with a serial loop
// took 29 us per operand at 8192^3.)  Block 0 also writes the product plan:
// output 0 = H_A H_B^T; output 1 = H_A Lo_B^T + Lo_A H_B^T.
__global__ __launch_bounds__(256) void accu_rowsum_pair_kernel(const int32_t* __restrict__ psumA, int m_pad,
                                                                int32_t* __restrict__ RS,
                                                                const int32_t* __restrict__ psumB, int n_pad,
                                                                int32_t* __restrict__ CS, int nchunks, int ga,
                                                                int4* __restrict__ plan) {
  __shared__ int part[4][64];
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    plan[0] = make_int4(0, 0, 1, 0);
    plan[1] = make_int4(0, 1, 2, 1);
  }
  const bool is_a = (int)blockIdx.x < ga;
  const int32_t* psum = is_a ? psumA : psumB;
  const int rows_pad = is_a ? m_pad : n_pad;
  const int lr = threadIdx.x & 63, g = threadIdx.x >> 6;
  const int r = (is_a ? blockIdx.x : blockIdx.x - ga) * 64 + lr;
  int v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (r < rows_pad) {
    int c = g;
    for (; c + 28 < nchunks; c += 32)
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] += psum[(long)(c + 4 * u) * rows_pad + r];
    for (; c < nchunks; c += 4) v[0] += psum[(long)c * rows_pad + r];
  }
#pragma unroll
  for (int u = 1; u < 8; ++u) v[0] += v[u];
  part[g][lr] = v[0];
  __syncthreads();
  if (g == 0 && r < rows_pad) (is_a ? RS : CS)[r] = part[0][lr] + part[1][lr] + part[2][lr] + part[3][lr];
}

__device__ __forceinline__ int block_reduce(int v, bool take_max, int* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int o = 32; o > 0; o >>= 1) {
    const int w = __shfl_xor(v, o, 64);
    v = take_max ? max(v, w) : min(v, w);
  }
  if (lane == 0) red[wave] = v;
  __syncthreads();
  v = red[0];
  for (int w = 1; w < (int)(blockDim.x >> 6); ++w) v = take_max ? max(v, red[w]) : min(v, red[w]);
  return v;
}

// Column j (one block): L_ij = K2 - floor(log2(V / N_ij)) from the two product
// planes and the Lo sums, and the column's first bit count
// b1_j = min(KMAX, floor((K2 - max_i L_ij) / 2)).
__global__ __launch_bounds__(256) void accu_combine_kernel(const int32_t* __restrict__ P, int m, int m_pad, long plane,
                                                            const int32_t* __restrict__ RS,
                                                            const int32_t* __restrict__ CS, int K2, int kmax,
                                                            uint64_t vtop, int bv, int8_t* __restrict__ L,
                                                            int32_t* __restrict__ b1) {
  __shared__ int red[4];
  const int j = blockIdx.x;
  const long col = (long)j * m_pad;
  const int cs = CS[j];
  int mx = LZERO;
  for (int i = threadIdx.x; i < m; i += 256) {
    const long long N = ((long long)P[col + i] << 14) + ((long long)P[plane + col + i] << 7) +
                        (long long)RES * min(RS[i], cs);
    const int l = N > 0 ? K2 - floor_log2_ratio((uint64_t)N, vtop, bv) : LZERO;
    L[col + i] = (int8_t)l;
    mx = max(mx, l);
  }
  mx = block_reduce(mx, true, red);
  if (threadIdx.x == 0) b1[j] = min(kmax, (K2 - mx) >> 1);  // arithmetic shift: floor
}

// Partial row minima of K2 - L_ij - b1_j over a chunk of CHUNK columns: 64
// rows per block, four threads per row each taking every fourth column
// (eight loads in flight), combined through LDS.  (One thread per row over
// the whole chunk, 256 dependent-issue loads, took 21.8 us at 1024^3.)
__global__ __launch_bounds__(256) void accu_rowmin_kernel(const int8_t* __restrict__ L, int m, int n, int m_pad,
                                                           const int32_t* __restrict__ b1, int K2,
                                                           int32_t* __restrict__ pmin) {
  __shared__ int bs[CHUNK];
  __shared__ int part[4][64];
  const int j0 = blockIdx.y * CHUNK;
  const int jn = min(CHUNK, n - j0);
  for (int t = threadIdx.x; t < jn; t += 256) bs[t] = b1[j0 + t];
  __syncthreads();
  const int r = threadIdx.x & 63, g = threadIdx.x >> 6;
  const int i = blockIdx.x * 64 + r;
  int v[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) v[u] = 1 << 30;
  if (i < m) {
    const int8_t* col = L + (long)j0 * m_pad + i;
    int t = g;
    for (; t + 28 < jn; t += 32)
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = min(v[u], K2 - (int)col[(long)(t + 4 * u) * m_pad] - bs[t + 4 * u]);
    for (; t < jn; t += 4) v[0] = min(v[0], K2 - (int)col[(long)t * m_pad] - bs[t]);
  }
#pragma unroll
  for (int u = 1; u < 8; ++u) v[0] = min(v[0], v[u]);
  part[g][r] = v[0];
  __syncthreads();
  if (g == 0 && i < m)
    pmin[(long)blockIdx.y * m_pad + i] = min(min(part[0][r], part[1][r]), min(part[2][r], part[3][r]));
}

// Row bit counts a_i and exponents e'_i (in place).
__global__ __launch_bounds__(256) void accu_rowfinal_kernel(const int32_t* __restrict__ pmin, int m, int m_pad,
                                                             int nchunks, int kmax, int32_t* __restrict__ a,
                                                             int32_t* __restrict__ e) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= m) return;
  int v = kmax;
  for (int c = 0; c < nchunks; ++c) v = min(v, pmin[(long)c * m_pad + i]);
  a[i] = v;
  const int ei = e[i];
  e[i] = ei == OZGEMM_EXP_NONFINITE ? ei : kmax - v + ei;
}

// Column j (one block): b_j = min(KMAX, min_i (K2 - L_ij - a_i)) and f'_j (in place).
__global__ __launch_bounds__(256) void accu_colfinal_kernel(const int8_t* __restrict__ L, int m, int m_pad,
                                                             const int32_t* __restrict__ a, int K2, int kmax,
                                                             int32_t* __restrict__ f) {
  __shared__ int red[4];
  const int j = blockIdx.x;
  const long col = (long)j * m_pad;
  int v = kmax;
  // four consecutive rows per thread and step, so that both loads stay
  // contiguous across the lanes: 4 bytes of L and 16 of a (both allocated
  // to m_pad entries, so whole groups stay in bounds; rows >= m are
  // skipped).  Byte loads, one row per thread and step, took 47 us at
  // 8192^3; 16 rows per thread (a read at a 64-byte lane stride) 56 us.
#pragma unroll 4
  for (int i0 = threadIdx.x * 4; i0 < m; i0 += 256 * 4) {
    const uint32_t lw = *reinterpret_cast<const uint32_t*>(L + col + i0);
    const int4 av = *reinterpret_cast<const int4*>(a + i0);
    const int aa[4] = {av.x, av.y, av.z, av.w};
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int li = (int)(int8_t)(lw >> (8 * b));
      if (i0 + b < m) v = min(v, K2 - li - aa[b]);
    }
  }
  v = block_reduce(v, false, red);
  if (threadIdx.x == 0) {
    const int fj = f[j];
    f[j] = fj == OZGEMM_EXP_NONFINITE ? fj : kmax - v + fj;
  }
}

}  // namespace

size_t accu_scratch_bytes(int m_pad, int n_pad, int q_pad) {
  const size_t mp = (size_t)m_pad, np = (size_t)n_pad;
  const size_t chunks = (np + CHUNK - 1) / CHUNK;
  return round_up(8 * mp * np, 256) + round_up(mp * np, 256) + round_up(4 * mp, 256) * 2 +
         round_up(4 * np, 256) * 2 + round_up(4 * chunks * mp, 256) + round_up((size_t)(q_pad / TK) * 4 * np, 256) +
         256;
}

hipError_t launch_accu_exponents(const double* A, int m, int q, int lda, const double* B, int n, int ldb, int m_pad,
                                 int n_pad, int q_pad, int K2, uint64_t vtop, int bv, int kmax, int8_t* Aplanes,
                                 int8_t* Bplanes, int32_t* psumA, char* scratch, int32_t* e, int32_t* f,
                                 hipStream_t st) {
  if (m < 1 || n < 1 || q < 1 || q_pad % TK || m_pad % 256 || n_pad % 256 || m_pad / TR > 65535 ||
      n_pad / TR > 65535 || q_pad > ACCU_Q_MAX || 2L * RES * RES * q_pad >= (1L << 31) || kmax != ACCU_KMAX ||
      bv < 64 || (vtop >> 63) == 0)
    return hipErrorInvalidValue;
  const size_t mp = (size_t)m_pad, np = (size_t)n_pad;
  const int nk = q_pad / TK;
  const int chunks = (n + CHUNK - 1) / CHUNK;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* p = scratch + off;
    off = round_up(off + bytes, 256);
    return p;
  };
  int32_t* P = reinterpret_cast<int32_t*>(take(8 * mp * np));  // two int32 planes [o][j][i]
  int8_t* L = reinterpret_cast<int8_t*>(take(mp * np));
  int32_t* RS = reinterpret_cast<int32_t*>(take(4 * mp));
  int32_t* a = reinterpret_cast<int32_t*>(take(4 * mp));
  int32_t* CS = reinterpret_cast<int32_t*>(take(4 * np));
  int32_t* b1 = reinterpret_cast<int32_t*>(take(4 * np));
  int32_t* pmin = reinterpret_cast<int32_t*>(take(4 * (size_t)chunks * mp));
  int32_t* psumB = reinterpret_cast<int32_t*>(take((size_t)nk * 4 * np));
  int4* plan = reinterpret_cast<int4*>(take(2 * sizeof(int4)));

  // bands of A's rows (A column-major: rows contiguous) and of B's columns,
  // then their Lo row sums and the product plan: two launches
  const long na = (long)nk * (m_pad / TR), nb = (long)nk * (n_pad / TR);
  if (na + nb > 0x7fffffffL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(accu_band_pair_kernel, dim3((unsigned)(na + nb)), dim3(256), 0, st, A, m, (long)lda, e, Aplanes,
                     Aplanes + mp * q_pad, m_pad, psumA, B, n, (long)ldb, f, Bplanes, Bplanes + np * q_pad, n_pad,
                     psumB, q, q_pad, (int)na);
  hipLaunchKernelGGL(accu_rowsum_pair_kernel, dim3(m_pad / 64 + n_pad / 64), dim3(256), 0, st, psumA, m_pad, RS,
                     psumB, n_pad, CS, nk, m_pad / 64, plan);
  hipError_t err = launch_gemm_multi(Aplanes, Bplanes, m_pad, n_pad, q_pad, plan, 2, P, st);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(accu_combine_kernel, dim3(n), dim3(256), 0, st, P, m, m_pad, (long)(mp * np), RS, CS, K2, kmax,
                     vtop, bv, L, b1);
  hipLaunchKernelGGL(accu_rowmin_kernel, dim3((m + 63) / 64, chunks), dim3(256), 0, st, L, m, n, m_pad, b1, K2,
                     pmin);
  hipLaunchKernelGGL(accu_rowfinal_kernel, dim3((m + 255) / 256), dim3(256), 0, st, pmin, m, m_pad, chunks, kmax, a,
                     e);
  hipLaunchKernelGGL(accu_colfinal_kernel, dim3(n), dim3(256), 0, st, L, m, m_pad, a, K2, kmax, f);
  return hipGetLastError();
}

}  // namespace oz
