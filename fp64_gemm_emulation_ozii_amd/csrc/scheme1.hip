// Scheme I on int8 matrix cores: slice split and FP64 accumulation kernels.
//
// Ozaki I notes, optimized algorithm (after Uchino, Ozaki and Imamura):
//  * RN split: slice p of a row is its residual rounded to the grid
//    mu = 2^(ceil(log2 max|residual|) + 1 - beta), ties to even; the integer
//    rint(residual / mu) fits in [-2^(beta-1), 2^(beta-1)];
//  * Hybrid split: the grid of slice p is mu'' 2^(-beta (p-1)) with mu'' taken
//    once from the original row maximum;
//  * products A_i B_j for i + j <= k + 1, each or (for Hybrid) runs of r with
//    the same i + j summed exactly in int32 (the shared GEMM kernel), then
//    converted to FP64, scaled by the power-of-two grids and added to C in a
//    fixed order (i-major, j-minor; or by increasing i + j).
//
// Every step is exact except the FP64 additions of the accumulation, which
// are done in the documented order, so the result is reproducible bit for
// bit.  Grids are kept as int32 exponents g (mu = 2^g); a row holding Inf or
// NaN is flagged by OZGEMM_EXP_NONFINITE in its first grid exponent and is
// split as zero.
#include "oz_internal.h"

namespace oz {

namespace {

constexpr int TR = 32;              // rows per split tile
constexpr int TK = 128;             // inner-dimension entries per split tile
constexpr int LDS_STRIDE = TK + 1;  // doubles; odd stride spreads banks

// ceil(log2 x) of a finite positive double given by its bit pattern.
__device__ __forceinline__ int ceil_log2_bits(uint64_t b) {
  const int ex = (int)(b >> 52);
  const uint64_t man = b & ((1ull << 52) - 1);
  if (ex == 0) {  // subnormal: man * 2^-1074
    const int top = 63 - __builtin_clzll(man);
    return top - 1074 + (((man & (man - 1)) != 0) ? 1 : 0);
  }
  return ex - 1023 + (man != 0 ? 1 : 0);
}

// The residual after rounding a to the grid 2^g: returns n = rint(a 2^-g)
// and replaces a by a - n 2^g, exactly.  For n != 0, |a 2^-g| >= 1/2, so the
// scaling is exact and the difference is formed on the grid as
// (a 2^-g - n) 2^g, which stays finite where n 2^g alone would overflow (a
// row maximum within one grid step of the largest double).  For n = 0 the
// residual is a (a 2^-g may have lost bits to underflow there).
__device__ __forceinline__ double peel(double& a, int g) {
  const double x = __builtin_ldexp(a, -g);
  const double nn = __builtin_rint(x);
  a = (nn == 0.0) ? a : __builtin_ldexp(x - nn, g);
  return nn;
}

// MODE 0: partial row maxima of |X| (bit patterns, non-finite values kept).
// MODE 1: RN split pass `pass`: slice `pass` into its plane and, when
//         another pass follows, partial row maxima of the new residual.
// MODE 2: Hybrid split: all k slices.
// Element (r, l) of X sits at X[r*rs + l*ls]; each block converts a tile of
// TR rows x TK entries staged through LDS (coalesced for either layout).
template <bool ROWS_CONTIG, int MODE>
__global__ __launch_bounds__(256) void s1_split_kernel(const double* __restrict__ X, int rows, int q, long rs, long ls,
                                                        const int32_t* __restrict__ g, int rows_pad, int pass, int k,
                                                        int beta, int8_t* __restrict__ planes, long plane_stride,
                                                        int q_pad, uint64_t* __restrict__ pmax) {
  __shared__ double tile[TR * LDS_STRIDE];
  const int tid = threadIdx.x;
  const int r0 = blockIdx.y * TR;
  const int l0 = blockIdx.x * TK;

  // all loads in flight before any is used; out-of-range lanes read a
  // clamped valid element and store zero (q >= 1; no rows: zero tile)
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

  const int r = tid >> 3;           // 0..31
  const int cseg = (tid & 7) * 16;  // 0..112
  const int grow = r0 + r;          // < rows_pad (grid covers rows_pad / TR)

  double a[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) a[j] = tile[r * LDS_STRIDE + cseg + j];

  uint64_t mx = 0;
  if (MODE == 0) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint64_t b = (uint64_t)__double_as_longlong(a[j]) & 0x7fffffffffffffffull;
      mx = b > mx ? b : mx;
    }
  } else {
    const int g0 = g[grow];
    const bool bad = (g0 == OZGEMM_EXP_NONFINITE);
#pragma unroll
    for (int j = 0; j < 16; ++j) a[j] = bad ? 0.0 : a[j];
    if (MODE == 1) {
      for (int t = 0; t < pass; ++t) {
        const int gt = (t == 0 && bad) ? 0 : g[(long)t * rows_pad + grow];
#pragma unroll
        for (int j = 0; j < 16; ++j) (void)peel(a[j], gt);
      }
      const int gp = (pass == 0 && bad) ? 0 : g[(long)pass * rows_pad + grow];
      uint32_t packed[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int nn = (int)peel(a[j], gp);
        packed[j >> 2] |= ((uint32_t)nn & 0xffu) << (8 * (j & 3));
        const uint64_t b = (uint64_t)__double_as_longlong(a[j]) & 0x7fffffffffffffffull;
        mx = b > mx ? b : mx;
      }
      *reinterpret_cast<uint4*>(planes + (long)pass * plane_stride + (long)grow * q_pad + l0 + cseg) =
          make_uint4(packed[0], packed[1], packed[2], packed[3]);
    } else {
      const int gb = bad ? 0 : g0;
      for (int p = 0; p < k; ++p) {
        const int gp = gb - beta * p;
        uint32_t packed[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int nn = (int)peel(a[j], gp);
          packed[j >> 2] |= ((uint32_t)nn & 0xffu) << (8 * (j & 3));
        }
        *reinterpret_cast<uint4*>(planes + (long)p * plane_stride + (long)grow * q_pad + l0 + cseg) =
            make_uint4(packed[0], packed[1], packed[2], packed[3]);
      }
    }
  }

  if (pmax != nullptr && MODE != 2) {
    // the 8 threads of a row are 8 consecutive lanes of one wavefront
#pragma unroll
    for (int off = 1; off < 8; off <<= 1) {
      const uint64_t o = (uint64_t)__shfl_xor((long long)mx, off, 64);
      mx = o > mx ? o : mx;
    }
    if ((tid & 7) == 0) pmax[(long)blockIdx.x * rows_pad + grow] = mx;
  }
}

// One pass for a row held in LDS (the rows of B: a column of B is
// contiguous), for OZGEMM_ONE_PASS_Q_MIN <= q <= OZGEMM_ONE_PASS_Q_MAX.  The
// block loads the row, takes its maximum for the first grid, then writes the
// k slices in one sweep; with the RN split the grid of slice p + 1 comes from
// a block reduction of the residual left by slice p.  Grids, slices and the
// non-finite and padding cases are those of the rowmax + grid + split passes
// above (one pad double after every 16 entries keeps the 16-entry reads
// conflict-free; each thread keeps its two segments in registers).
constexpr int ROW_QMAX = OZGEMM_ONE_PASS_Q_MAX;
constexpr int ROW_LDS = ROW_QMAX + ROW_QMAX / 16;

template <int MODE>  // 1: RN, 2: Hybrid
__global__ __launch_bounds__(256) void s1_row_split_kernel(const double* __restrict__ X, int rows, int q, long rs,
                                                            int rows_pad, int q_pad, int k, int beta,
                                                            int32_t* __restrict__ g, int8_t* __restrict__ planes,
                                                            long plane_stride) {
  __shared__ double row[ROW_LDS];
  __shared__ uint64_t wmax[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rr = blockIdx.x;
  const bool live = rr < rows;  // uniform across the block
  uint64_t mx = 0;
  if (live) {
    const double* src = X + (long)rr * rs;
    double v[ROW_QMAX / 256];
#pragma unroll
    for (int i = 0; i < ROW_QMAX / 256; ++i) {
      const int l = tid + 256 * i;
      v[i] = l < q ? src[l] : 0.0;
    }
#pragma unroll
    for (int i = 0; i < ROW_QMAX / 256; ++i) {
      const int l = tid + 256 * i;
      mx = umax64(mx, abs_bits(v[i]));
      row[l + (l >> 4)] = v[i];
    }
  }
  // maximum over the block (every thread calls it; it also orders the LDS)
  auto block_max = [&](uint64_t x) -> uint64_t {
    for (int off = 32; off > 0; off >>= 1) x = umax64(x, (uint64_t)__shfl_xor((unsigned long long)x, off, 64));
    __syncthreads();  // the previous reduction's readers are done with wmax
    if (lane == 0) wmax[wave] = x;
    __syncthreads();
    return umax64(umax64(wmax[0], wmax[1]), umax64(wmax[2], wmax[3]));
  };
  auto grid_of = [&](uint64_t b) -> int {  // as s1_grid_kernel
    if (b >= 0x7ff0000000000000ull) return OZGEMM_EXP_NONFINITE;
    return b == 0 ? 0 : ceil_log2_bits(b) + 1 - beta;
  };
  const int g0 = grid_of(block_max(mx));
  const bool bad = (g0 == OZGEMM_EXP_NONFINITE);
  if (tid == 0) g[rr] = g0;

  constexpr int NSEG = ROW_QMAX / 16 / 256;  // 16-entry segments per thread
  double a[NSEG][16];
#pragma unroll
  for (int u = 0; u < NSEG; ++u) {
    const int seg = tid + 256 * u;
#pragma unroll
    for (int jj = 0; jj < 16; ++jj)
      a[u][jj] = (live && !bad && 16 * seg < q_pad) ? row[17 * seg + jj] : 0.0;  // entry 16 seg + jj
  }
  int gp = bad ? 0 : g0;
  for (int p = 0; p < k; ++p) {
    if (MODE == 2) gp = (bad ? 0 : g0) - beta * p;
    uint64_t rmx = 0;
#pragma unroll
    for (int u = 0; u < NSEG; ++u) {
      const int seg = tid + 256 * u;
      if (16 * seg >= q_pad) continue;
      uint32_t packed[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) {
        const int nn = (int)peel(a[u][jj], gp);
        packed[jj >> 2] |= ((uint32_t)nn & 0xffu) << (8 * (jj & 3));
        if (MODE == 1) rmx = umax64(rmx, abs_bits(a[u][jj]));
      }
      *reinterpret_cast<uint4*>(planes + (long)p * plane_stride + (long)rr * q_pad + 16 * seg) =
          make_uint4(packed[0], packed[1], packed[2], packed[3]);
    }
    if (MODE == 1 && p + 1 < k) {
      gp = grid_of(block_max(rmx));
      if (tid == 0) g[(long)(p + 1) * rows_pad + rr] = gp;
    }
  }
}

// Grid exponent of each row from the partial maxima: E + 1 - beta with
// E = ceil(log2 max); 0 for a zero row; OZGEMM_EXP_NONFINITE when the row
// holds Inf or NaN.
__global__ __launch_bounds__(256) void s1_grid_kernel(const uint64_t* __restrict__ pmax, int rows_pad, int nchunks,
                                                       int beta, int32_t* __restrict__ gout) {
  // 64 rows per block, four threads per row over every fourth chunk
  __shared__ uint64_t part[4][64];
  const int r = threadIdx.x & 63, gi = threadIdx.x >> 6;
  const int row = blockIdx.x * 64 + r;
  uint64_t v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (row < rows_pad) {
    int c = gi;
    for (; c + 28 < nchunks; c += 32)
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint64_t x = pmax[(long)(c + 4 * u) * rows_pad + row];
        v[u] = x > v[u] ? x : v[u];
      }
    for (; c < nchunks; c += 4) {
      const uint64_t x = pmax[(long)c * rows_pad + row];
      v[0] = x > v[0] ? x : v[0];
    }
  }
#pragma unroll
  for (int u = 1; u < 8; ++u) v[0] = v[u] > v[0] ? v[u] : v[0];
  part[gi][r] = v[0];
  __syncthreads();
  if (gi != 0 || row >= rows_pad) return;
  uint64_t mx = part[0][r];
#pragma unroll
  for (int u = 1; u < 4; ++u) mx = part[u][r] > mx ? part[u][r] : mx;
  int gv;
  if (mx >= 0x7ff0000000000000ull) gv = OZGEMM_EXP_NONFINITE;
  else if (mx == 0) gv = 0;
  else gv = ceil_log2_bits(mx) + 1 - beta;
  gout[row] = gv;
}

// C_ij = sum over the accumulation plan, in its order, of
// ldexp(P_o[j][i], gA[plan.x][i] + gB[plan.y][j] + plan.z); NaN where row i
// of A or column j of B is flagged non-finite.  Thread = 4 consecutive rows
// of one column (one 16-byte load per product plane).
__global__ __launch_bounds__(256) void s1_accum_kernel(const int32_t* __restrict__ P, int m, int n, int m_pad,
                                                        long plane, int nout, const int4* __restrict__ acc,
                                                        const int32_t* __restrict__ gA, int ma_pad,
                                                        const int32_t* __restrict__ gB, int nb_pad,
                                                        double* __restrict__ C, long ldc) {
  const int i0 = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (i0 >= m) return;
  const int4 bad_a = *reinterpret_cast<const int4*>(gA + i0);
  const bool ba[4] = {bad_a.x == OZGEMM_EXP_NONFINITE, bad_a.y == OZGEMM_EXP_NONFINITE,
                      bad_a.z == OZGEMM_EXP_NONFINITE, bad_a.w == OZGEMM_EXP_NONFINITE};
  for (int j = blockIdx.y; j < n; j += gridDim.y) {
    const bool bb = gB[j] == OZGEMM_EXP_NONFINITE;
    double c[4] = {0.0, 0.0, 0.0, 0.0};
    // four product planes per round: their loads are issued together, the
    // additions stay in plan order
    for (int o0 = 0; o0 < nout; o0 += 4) {
      int4 v[4], ea[4];
      int eb[4];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const int4 pl = acc[min(o0 + d, nout - 1)];
        v[d] = *reinterpret_cast<const int4*>(P + (long)pl.w * plane + (long)j * m_pad + i0);
        ea[d] = *reinterpret_cast<const int4*>(gA + (long)pl.x * ma_pad + i0);
        eb[d] = gB[(long)pl.y * nb_pad + j] + pl.z;
      }
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        if (o0 + d >= nout) break;  // uniform
        const int vv[4] = {v[d].x, v[d].y, v[d].z, v[d].w};
        const int ee[4] = {ea[d].x, ea[d].y, ea[d].z, ea[d].w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int e = (ba[u] || bb) ? 0 : ee[u] + eb[d];
          c[u] = c[u] + __builtin_ldexp((double)vv[u], e);
        }
      }
    }
    double* out = C + (long)j * ldc + i0;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (i0 + u < m) out[u] = (ba[u] || bb) ? __builtin_nan("") : c[u];
  }
}

// Builds the product plan (GEMM side) and the accumulation plan on the
// device, so that a call needs no host-to-device copy.
//   RN:     output o = o-th pair (i, j) of the triangle, i-major, j-minor;
//           GEMM {i-1, j-1, 1, o}; accumulation {i-1, j-1, 0, o}.
//   Hybrid: output o = o-th run of at most r pairs (s, g-s), s increasing,
//           for g = 2..k+1; GEMM {s0-1, g-s0-1, len, o};
//           accumulation {0, 0, -beta (g-2), o}.
// GEMM entries are ordered by decreasing run length (longest first).
__global__ void s1_plan_kernel(int variant, int k, int r, int beta, int4* gemm_plan, int4* acc_plan) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  int o = 0;
  if (variant == OZGEMM_S1_RN) {
    for (int i = 1; i <= k; ++i)
      for (int j = 1; j <= k - i + 1; ++j) {
        gemm_plan[o] = make_int4(i - 1, j - 1, 1, o);
        acc_plan[o] = make_int4(i - 1, j - 1, 0, o);
        ++o;
      }
    return;
  }
  for (int gg = 2; gg <= k + 1; ++gg) {
    int s0 = 1;
    while (s0 <= gg - 1) {
      const int len = min(r, gg - s0);
      gemm_plan[o] = make_int4(s0 - 1, gg - s0 - 1, len, o);
      acc_plan[o] = make_int4(0, 0, -beta * (gg - 2), o);
      ++o;
      s0 += len;
    }
  }
  // longest runs first for the GEMM grid (stable insertion sort, o <= 136)
  for (int x = 1; x < o; ++x) {
    const int4 v = gemm_plan[x];
    int y = x - 1;
    while (y >= 0 && gemm_plan[y].z < v.z) {
      gemm_plan[y + 1] = gemm_plan[y];
      --y;
    }
    gemm_plan[y + 1] = v;
  }
}

}  // namespace

hipError_t launch_s1_rowmax(const double* X, int rows, int q, long rs, long ls, int rows_pad, int q_pad,
                            uint64_t* pmax, hipStream_t st) {
  if (rows_pad / TR > 65535) return hipErrorInvalidValue;  // grid.y
  const dim3 grid(q_pad / TK, rows_pad / TR);
  if (rs == 1)
    hipLaunchKernelGGL((s1_split_kernel<true, 0>), grid, dim3(256), 0, st, X, rows, q, rs, ls, nullptr, rows_pad, 0,
                       0, 0, nullptr, 0L, q_pad, pmax);
  else
    hipLaunchKernelGGL((s1_split_kernel<false, 0>), grid, dim3(256), 0, st, X, rows, q, rs, ls, nullptr, rows_pad, 0,
                       0, 0, nullptr, 0L, q_pad, pmax);
  return hipGetLastError();
}

hipError_t launch_s1_grid(const uint64_t* pmax, int rows_pad, int nchunks, int beta, int32_t* gout,
                          hipStream_t st) {
  hipLaunchKernelGGL(s1_grid_kernel, dim3((rows_pad + 63) / 64), dim3(256), 0, st, pmax, rows_pad, nchunks, beta,
                     gout);
  return hipGetLastError();
}

hipError_t launch_s1_split(const double* X, int rows, int q, long rs, long ls, const int32_t* g, int rows_pad,
                           int q_pad, int variant, int pass, int k, int beta, int8_t* planes, uint64_t* pmax,
                           hipStream_t st) {
  if (rows_pad / TR > 65535) return hipErrorInvalidValue;  // grid.y
  const dim3 grid(q_pad / TK, rows_pad / TR);
  const long plane_stride = (long)rows_pad * q_pad;
#define OZ_S1_LAUNCH(RC, MD)                                                                                 \
  hipLaunchKernelGGL((s1_split_kernel<RC, MD>), grid, dim3(256), 0, st, X, rows, q, rs, ls, g, rows_pad, pass, \
                     k, beta, planes, plane_stride, q_pad, pmax)
  if (variant == OZGEMM_S1_RN) {
    if (rs == 1) OZ_S1_LAUNCH(true, 1);
    else OZ_S1_LAUNCH(false, 1);
  } else {
    if (rs == 1) OZ_S1_LAUNCH(true, 2);
    else OZ_S1_LAUNCH(false, 2);
  }
#undef OZ_S1_LAUNCH
  return hipGetLastError();
}

bool s1_row_split_fits(int q) { return q >= OZGEMM_ONE_PASS_Q_MIN && q <= ROW_QMAX; }

hipError_t launch_s1_row_split(const double* X, int rows, int q, long rs, int rows_pad, int q_pad, int variant, int k,
                               int beta, int32_t* g, int8_t* planes, hipStream_t st) {
  if (!s1_row_split_fits(q) || q_pad > ROW_QMAX || q_pad % 16 || rows_pad < rows) return hipErrorInvalidValue;
  const long plane_stride = (long)rows_pad * q_pad;
  if (variant == OZGEMM_S1_RN)
    hipLaunchKernelGGL((s1_row_split_kernel<1>), dim3(rows_pad), dim3(256), 0, st, X, rows, q, rs, rows_pad, q_pad,
                       k, beta, g, planes, plane_stride);
  else
    hipLaunchKernelGGL((s1_row_split_kernel<2>), dim3(rows_pad), dim3(256), 0, st, X, rows, q, rs, rows_pad, q_pad,
                       k, beta, g, planes, plane_stride);
  return hipGetLastError();
}

hipError_t launch_s1_plan(int variant, int k, int r, int beta, int4* gemm_plan, int4* acc_plan, hipStream_t st) {
  hipLaunchKernelGGL(s1_plan_kernel, dim3(1), dim3(64), 0, st, variant, k, r, beta, gemm_plan, acc_plan);
  return hipGetLastError();
}

hipError_t launch_s1_accum(const int32_t* P, int m, int n, int m_pad, int n_pad, int nout, const int4* acc,
                           const int32_t* gA, int ma_pad, const int32_t* gB, int nb_pad, double* C, int ldc,
                           hipStream_t st) {
  const dim3 grid((m + 1023) / 1024, std::min(n, 65535));
  hipLaunchKernelGGL(s1_accum_kernel, grid, dim3(256), 0, st, P, m, n, m_pad, (long)m_pad * n_pad, nout, acc, gA,
                     ma_pad, gB, nb_pad, C, (long)ldc);
  return hipGetLastError();
}

}  // namespace oz
