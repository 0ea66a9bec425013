// Scale step: per-row exponents of A and per-column exponents of B.
//
// Ozaki II notes §3: D and E are diagonal powers of two; §5: keeping k bits
// needs |a_il 2^(k - e_i)| < 2^k.  e_i is the frexp exponent of the row
// maximum: 2^(e_i - 1) <= max_l |a_il| < 2^e_i.
//
// The maxima are taken on the IEEE bit patterns with the sign cleared: for
// non-negative doubles the unsigned integer order is the numeric order, and
// Inf/NaN patterns (>= 0x7ff0...) sort above every finite value, so a
// non-finite row is recognised from its maximum alone.
//
// A is column-major, so a row is strided: one thread per row walks a chunk of
// columns (consecutive threads read consecutive rows -> coalesced), the
// chunks are combined by a second small kernel.  A column of B is
// contiguous: one wavefront per column, then a cross-lane reduction.
//
// OS II-fast budget (Ozaki II notes §9: a Cauchy-Schwarz bound of c_max):
// a second pass bounds each row norm, S_i = sum_l ceil(|a_il| 2^(20 - e_i))^2
// (an exact integer, at most q 2^40, so the order of the additions does not
// matter), and replaces e_i by e'_i = kb - d_i with the row shift
// d_i = kappa - c_i - e_i, 4^c_i the smallest power of four >= S_i 2^-40.
// Then ||trunc(a_i 2^d_i)|| <= 2^kappa, and the residue and CRT kernels use
// e'_i exactly like e_i (shift kb - e'_i, unscale e'_i + f'_j - 2 kb).
#include "oz_internal.h"

namespace oz {

// Block (bx, by) of the partial row maxima: rows bx*256.., columns by*chunk..
__device__ __forceinline__ void row_max_partial_block(const double* __restrict__ A, int m, int q, long lda,
                                                      int chunk, uint64_t* __restrict__ pmax, int m_stride, int bx,
                                                      int by) {
  const int i = bx * 256 + threadIdx.x;
  const int l0 = by * chunk;
  const int l1 = min(q, l0 + chunk);
  uint64_t v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (i < m) {
    const double* p = A + i + (long)l0 * lda;
    int l = l0;
    for (; l + 8 <= l1; l += 8) {  // eight independent loads in flight
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = umax64(v[u], abs_bits(__builtin_nontemporal_load(p + u * lda)));
      p += 8 * lda;
    }
    for (; l < l1; ++l) {
      v[0] = umax64(v[0], abs_bits(*p));
      p += lda;
    }
  }
#pragma unroll
  for (int u = 1; u < 8; ++u) v[0] = umax64(v[0], v[u]);
  pmax[(long)by * m_stride + i] = v[0];
}

__global__ __launch_bounds__(256) void row_max_partial_kernel(const double* __restrict__ A, int m, int q,
                                                               long lda, int chunk,
                                                               uint64_t* __restrict__ pmax, int m_stride) {
  row_max_partial_block(A, m, q, lda, chunk, pmax, m_stride, blockIdx.x, blockIdx.y);
}

// 64 rows per block, four threads per row each taking every fourth chunk
// (eight loads in flight), combined through LDS.
__global__ __launch_bounds__(256) void row_exp_finalize_kernel(const uint64_t* __restrict__ pmax, int m,
                                                                int m_stride, int nchunks,
                                                                int32_t* __restrict__ e) {
  __shared__ uint64_t part[4][64];
  const int r = threadIdx.x & 63, g = threadIdx.x >> 6;
  const int i = blockIdx.x * 64 + r;
  uint64_t v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (i < m) {
    int c = g;
    for (; c + 28 < nchunks; c += 32)
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = umax64(v[u], pmax[(long)(c + 4 * u) * m_stride + i]);
    for (; c < nchunks; c += 4) v[0] = umax64(v[0], pmax[(long)c * m_stride + i]);
  }
#pragma unroll
  for (int u = 1; u < 8; ++u) v[0] = umax64(v[0], v[u]);
  part[g][r] = v[0];
  __syncthreads();
  if (g == 0 && i < m)
    e[i] = exponent_of_bits(umax64(umax64(part[0][r], part[1][r]), umax64(part[2][r], part[3][r])));
}

// Block bx of the column maxima: columns 4 bx.., one wavefront each.
__device__ __forceinline__ void col_exp_block(const double* __restrict__ B, int q, int n, long ldb,
                                              int32_t* __restrict__ f, int bx) {
  const int lane = threadIdx.x & 63;
  const int j = bx * 4 + (threadIdx.x >> 6);
  if (j >= n) return;  // whole wavefront exits together
  const double* col = B + (long)j * ldb;
  uint64_t w[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  int l = lane;
  for (; l + 448 < q; l += 512)  // eight independent loads in flight
#pragma unroll
    for (int u = 0; u < 8; ++u) w[u] = umax64(w[u], abs_bits(__builtin_nontemporal_load(col + l + 64 * u)));
  for (; l < q; l += 64) w[0] = umax64(w[0], abs_bits(col[l]));
  uint64_t v = w[0];
#pragma unroll
  for (int u = 1; u < 8; ++u) v = umax64(v, w[u]);
  for (int off = 32; off > 0; off >>= 1) v = umax64(v, (uint64_t)__shfl_xor((unsigned long long)v, off, 64));
  if (lane == 0) f[j] = exponent_of_bits(v);
}

__global__ __launch_bounds__(256) void col_exp_kernel(const double* __restrict__ B, int q, int n, long ldb,
                                                       int32_t* __restrict__ f) {
  col_exp_block(B, q, n, ldb, f, blockIdx.x);
}

// A's partial row maxima and B's column maxima in one launch (they are
// independent): blocks [0, na) are row_max_partial_kernel's in row-major
// order of its (gxa x nchunks) grid, the rest col_exp_kernel's.  For small
// products the two kernels' ramp-up and drain then overlap.
__global__ __launch_bounds__(256) void scale_pair_kernel(const double* __restrict__ A, int m, int q, long lda,
                                                          int chunk, uint64_t* __restrict__ pmax, int m_stride,
                                                          int gxa, int na, const double* __restrict__ B, int n,
                                                          long ldb, int32_t* __restrict__ f) {
  const int b = blockIdx.x;
  if (b < na)
    row_max_partial_block(A, m, q, lda, chunk, pmax, m_stride, b % gxa, b / gxa);
  else
    col_exp_block(B, q, n, ldb, f, b - na);
}

// Block (bx, by) of the partial row norm bounds: rows bx*256.., columns by*chunk..
__device__ __forceinline__ void row_norm_partial_block(const double* __restrict__ A, int m, int q, long lda,
                                                       int chunk, const int32_t* __restrict__ e,
                                                       uint64_t* __restrict__ psum, int m_stride, int bx, int by) {
  const int i = bx * 256 + threadIdx.x;
  const int l0 = by * chunk;
  const int l1 = min(q, l0 + chunk);
  uint64_t v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (i < m) {
    const int ei = e[i];
    if (ei != OZGEMM_EXP_NONFINITE) {
      const double* p = A + i + (long)l0 * lda;
      int l = l0;
      for (; l + 8 <= l1; l += 8) {  // eight independent loads in flight (the sum is exact in any order)
        double x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) x[u] = __builtin_nontemporal_load(p + u * lda);
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] += norm_term(x[u], ei);
        p += 8 * lda;
      }
      for (; l < l1; ++l) {
        v[0] += norm_term(*p, ei);
        p += lda;
      }
    }
  }
#pragma unroll
  for (int u = 1; u < 8; ++u) v[0] += v[u];
  psum[(long)by * m_stride + i] = v[0];
}

__global__ __launch_bounds__(256) void row_norm_partial_kernel(const double* __restrict__ A, int m, int q,
                                                                long lda, int chunk,
                                                                const int32_t* __restrict__ e,
                                                                uint64_t* __restrict__ psum, int m_stride) {
  row_norm_partial_block(A, m, q, lda, chunk, e, psum, m_stride, blockIdx.x, blockIdx.y);
}

// Like row_exp_finalize_kernel: 64 rows per block, four threads per row
// each summing every fourth chunk (eight loads in flight), combined through
// LDS (one thread per row with a serial loop took 9.3 us at 1024^3 against
// 4 us for the row-exponent finalisation).
__global__ __launch_bounds__(256) void row_fast_finalize_kernel(const uint64_t* __restrict__ psum, int m,
                                                                 int m_stride, int nchunks, int kappa, int kb,
                                                                 int32_t* __restrict__ e) {
  __shared__ uint64_t part[4][64];
  const int r = threadIdx.x & 63, g = threadIdx.x >> 6;
  const int i = blockIdx.x * 64 + r;
  uint64_t v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (i < m) {
    int c = g;
    for (; c + 28 < nchunks; c += 32)
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] += psum[(long)(c + 4 * u) * m_stride + i];
    for (; c < nchunks; c += 4) v[0] += psum[(long)c * m_stride + i];
  }
#pragma unroll
  for (int u = 1; u < 8; ++u) v[0] += v[u];
  part[g][r] = v[0];
  __syncthreads();
  if (g == 0 && i < m) e[i] = fast_exponent(e[i], part[0][r] + part[1][r] + part[2][r] + part[3][r], kappa, kb);
}

// Block bx of the column norm bounds: columns 4 bx.., one wavefront each.
__device__ __forceinline__ void col_fast_block(const double* __restrict__ B, int q, int n, long ldb, int kappa,
                                               int kb, int32_t* __restrict__ f, int bx) {
  const int lane = threadIdx.x & 63;
  const int j = bx * 4 + (threadIdx.x >> 6);
  if (j >= n) return;  // whole wavefront exits together
  const int fj = f[j];
  uint64_t S = 0;
  if (fj != OZGEMM_EXP_NONFINITE) {
    const double* col = B + (long)j * ldb;
    uint64_t w[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    int l = lane;
    for (; l + 448 < q; l += 512) {  // eight independent loads in flight (the sum is exact in any order)
      double x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) x[u] = __builtin_nontemporal_load(col + l + 64 * u);
#pragma unroll
      for (int u = 0; u < 8; ++u) w[u] += norm_term(x[u], fj);
    }
    for (; l < q; l += 64) w[0] += norm_term(col[l], fj);
    S = w[0];
#pragma unroll
    for (int u = 1; u < 8; ++u) S += w[u];
    for (int off = 32; off > 0; off >>= 1) S += (uint64_t)__shfl_xor((unsigned long long)S, off, 64);
  }
  if (lane == 0) f[j] = fast_exponent(fj, S, kappa, kb);
}

__global__ __launch_bounds__(256) void col_fast_kernel(const double* __restrict__ B, int q, int n, long ldb,
                                                        int kappa, int kb, int32_t* __restrict__ f) {
  col_fast_block(B, q, n, ldb, kappa, kb, f, blockIdx.x);
}

// OS II-fast's partial row norm bounds of A and column bounds of B in one
// launch (independent, like scale_pair_kernel's two halves).
__global__ __launch_bounds__(256) void fast_pair_kernel(const double* __restrict__ A, int m, int q, long lda,
                                                         int chunk, const int32_t* __restrict__ e,
                                                         uint64_t* __restrict__ psum, int m_stride, int gxa, int na,
                                                         const double* __restrict__ B, int n, long ldb, int kappa_b,
                                                         int kb, int32_t* __restrict__ f) {
  const int b = blockIdx.x;
  if (b < na)
    row_norm_partial_block(A, m, q, lda, chunk, e, psum, m_stride, b % gxa, b / gxa);
  else
    col_fast_block(B, q, n, ldb, kappa_b, kb, f, b - na);
}

// The partial-sum kernels write one word per row of every 256-row block,
// padding rows included, into each of the nchunks rows of stride m_stride.
// q = 0 is valid: every row (column) then has the exponent of zero.
inline bool row_args_ok(int m, int q, int m_stride, int nchunks) {
  return m >= 1 && q >= 0 && nchunks >= 1 && nchunks <= 65535 && m_stride >= (m + 255) / 256 * 256;
}

hipError_t launch_row_max_partial(const double* A, int m, int q, int lda, uint64_t* pmax, int m_stride,
                                  int nchunks, hipStream_t st) {
  if (!row_args_ok(m, q, m_stride, nchunks)) return hipErrorInvalidValue;
  const int chunk = (q + nchunks - 1) / nchunks;
  dim3 grid((m + 255) / 256, nchunks);
  hipLaunchKernelGGL(row_max_partial_kernel, grid, dim3(256), 0, st, A, m, q, (long)lda, chunk, pmax, m_stride);
  return hipGetLastError();
}

hipError_t launch_row_exp_finalize(const uint64_t* pmax, int m, int m_stride, int nchunks, int32_t* e,
                                   hipStream_t st) {
  if (!row_args_ok(m, 1, m_stride, nchunks)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(row_exp_finalize_kernel, dim3((m + 63) / 64), dim3(256), 0, st, pmax, m, m_stride, nchunks,
                     e);
  return hipGetLastError();
}

hipError_t launch_scale_pair(const double* A, int m, int q, int lda, uint64_t* pmax, int m_stride, int nchunks,
                             const double* B, int n, int ldb, int32_t* f, hipStream_t st) {
  if (!row_args_ok(m, q, m_stride, nchunks) || n < 1) return hipErrorInvalidValue;
  const int chunk = (q + nchunks - 1) / nchunks;
  const int gxa = (m + 255) / 256, na = gxa * nchunks, nb = (n + 3) / 4;
  hipLaunchKernelGGL(scale_pair_kernel, dim3(na + nb), dim3(256), 0, st, A, m, q, (long)lda, chunk, pmax, m_stride,
                     gxa, na, B, n, (long)ldb, f);
  return hipGetLastError();
}

hipError_t launch_col_exp(const double* B, int q, int n, int ldb, int32_t* f, hipStream_t st) {
  if (n < 1 || q < 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(col_exp_kernel, dim3((n + 3) / 4), dim3(256), 0, st, B, q, n, (long)ldb, f);
  return hipGetLastError();
}

hipError_t launch_row_fast(const double* A, int m, int q, int lda, uint64_t* psum, int m_stride, int nchunks,
                           int kappa, int kb, int32_t* e, hipStream_t st) {
  if (!row_args_ok(m, q, m_stride, nchunks)) return hipErrorInvalidValue;
  const int chunk = (q + nchunks - 1) / nchunks;
  dim3 grid((m + 255) / 256, nchunks);
  hipLaunchKernelGGL(row_norm_partial_kernel, grid, dim3(256), 0, st, A, m, q, (long)lda, chunk, e, psum,
                     m_stride);
  hipLaunchKernelGGL(row_fast_finalize_kernel, dim3((m + 63) / 64), dim3(256), 0, st, psum, m, m_stride, nchunks,
                     kappa, kb, e);
  return hipGetLastError();
}

hipError_t launch_fast_pair(const double* A, int m, int q, int lda, uint64_t* psum, int m_stride, int nchunks,
                            int kappa_a, const double* B, int n, int ldb, int kappa_b, int kb, int32_t* e,
                            int32_t* f, hipStream_t st) {
  if (!row_args_ok(m, q, m_stride, nchunks) || n < 1) return hipErrorInvalidValue;
  const int chunk = (q + nchunks - 1) / nchunks;
  const int gxa = (m + 255) / 256, na = gxa * nchunks, nb = (n + 3) / 4;
  hipLaunchKernelGGL(fast_pair_kernel, dim3(na + nb), dim3(256), 0, st, A, m, q, (long)lda, chunk, e, psum,
                     m_stride, gxa, na, B, n, (long)ldb, kappa_b, kb, f);
  hipLaunchKernelGGL(row_fast_finalize_kernel, dim3((m + 63) / 64), dim3(256), 0, st, psum, m, m_stride, nchunks,
                     kappa_a, kb, e);
  return hipGetLastError();
}

hipError_t launch_col_fast(const double* B, int q, int n, int ldb, int kappa, int kb, int32_t* f, hipStream_t st) {
  if (n < 1 || q < 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(col_fast_kernel, dim3((n + 3) / 4), dim3(256), 0, st, B, q, n, (long)ldb, kappa, kb, f);
  return hipGetLastError();
}

}  // namespace oz
