// CRT reconstruction, range reduction and unscaling (one output per thread).
//
// Ozaki II notes §4: X = sum_t C''_t M_t y_t (mod M); §5: with 2 c_max < M
// the symmetric representative is the integer product A'B' itself;
// §7 steps 4-6: accumulate, reduce, unscale by D^-1 and E^-1.
//
// 1. S_l = sum_t r_t w_{t,l}, where w_{t,l} are the W-bit limbs of
//    W_t = M_t y_t (a small device table, staged in LDS per block).  With
//    W = 32 each term is < 2^40 and there are at most 20, so every partial
//    sum is below 2^45; with W = 40 (used while log2 M <= 120, s <= 15)
//    each term is < 2^48 and the sums stay below 2^52.  Either way the FP64
//    fused multiply-adds are exact.
// 2. The limb sums go to reconstruct40 or reconstruct_limbs
//    (crt_reconstruct.h): balanced carries, X = Z - Q M with
//    Q = rint(Z / M), one exact shift by M into (-M/2, M/2), and a single
//    rounding of X * 2^(e_i + f_j - 2k) to nearest-even (subnormal and
//    overflowing results included).
#include "oz_internal.h"

namespace oz {

namespace {

// Thread = 4 consecutive rows of one output column: the product residues of
// each modulus come in as one 32-bit load (the planes are padded to whole
// tiles, so rows up to the padded height are always readable), all s of them
// issued before the first is used.  The limbs of W_t sit in LDS, read once
// per modulus for all four rows.  NG = ceil(s / 4): only the last group of
// four moduli can be partial.
template <int L, bool W40, int NG>
__global__ __launch_bounds__(256) void crt_kernel(const uint8_t* __restrict__ rt, int m, int n, int m_pad,
                                                   long plane, const int32_t* __restrict__ e,
                                                   const int32_t* __restrict__ f, CrtConsts c,
                                                   double* __restrict__ C, long ldc) {
  __shared__ double wl[OZGEMM_S_MAX * MAX_LIMBS];
  for (int idx = threadIdx.x; idx < OZGEMM_S_MAX * MAX_LIMBS; idx += 256)
    wl[idx] = idx < c.s * MAX_LIMBS ? c.wtab[idx] : 0.0;
  __syncthreads();
  const int i0 = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (i0 >= m) return;
  const int s = c.s;
  int ei[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) ei[u] = e[min(i0 + u, m - 1)];
  // the residues of the next column this thread handles are loaded before
  // the current column is reduced, so their latency overlaps the arithmetic
  auto load_col = [&](int j, uint32_t* rr) {
    const uint8_t* p = rt + (long)j * m_pad + i0;
#pragma unroll
    for (int t = 0; t < 4 * NG; ++t)
      rr[t] = (t < 4 * (NG - 1) || t < s) ? *reinterpret_cast<const uint32_t*>(p + (long)t * plane) : 0u;
  };
  uint32_t rr[4 * NG], rn[4 * NG];
  if (blockIdx.y < n) load_col(blockIdx.y, rr);
  for (int j = blockIdx.y; j < n; j += gridDim.y) {
    const int fj = f[j];
    const int jn = j + gridDim.y;
    if (jn < n) load_col(jn, rn);
    // 1. exact FP64 limb sums for the four rows
    double S[4][L];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int l = 0; l < L; ++l) S[u][l] = 0.0;
#pragma unroll
    for (int t = 0; t < 4 * NG; ++t) {
      if (t >= 4 * (NG - 1) && t >= s) break;  // uniform: the last group may be partial
      double w[L];
#pragma unroll
      for (int l = 0; l < L; ++l) w[l] = wl[t * MAX_LIMBS + l];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const double r = (double)((rr[t] >> (8 * u)) & 0xffu);
#pragma unroll
        for (int l = 0; l < L; ++l) S[u][l] = __builtin_fma(r, w[l], S[u][l]);
      }
    }
    // 2. one row at a time (keeps the live registers of a single
    //    reconstruction, so more wavefronts fit on a SIMD)
    double* out = C + (long)j * ldc + i0;
    double res[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      res[u] = W40 ? reconstruct40<(L <= 3 ? L : 3)>(S[u], c.K, ei[u] + fj - 2 * c.k)
                   : reconstruct_limbs<L>(S[u], c.K, ei[u] + fj - 2 * c.k);
      if (ei[u] == OZGEMM_EXP_NONFINITE || fj == OZGEMM_EXP_NONFINITE) res[u] = __builtin_nan("");
      __builtin_amdgcn_sched_barrier(0);
    }
    // four rows as two 16-byte stores where the column allows it (the same
    // for every lane of a wave: i0 is a multiple of 4)
    if (i0 + 3 < m && ((reinterpret_cast<uintptr_t>(out) & 15) == 0)) {
      reinterpret_cast<double2*>(out)[0] = double2{res[0], res[1]};
      reinterpret_cast<double2*>(out)[1] = double2{res[2], res[3]};
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (i0 + u < m) out[u] = res[u];
    }
#pragma unroll
    for (int t = 0; t < 4 * NG; ++t) rr[t] = rn[t];
  }
}

__global__ void fill_zero_kernel(double* C, int m, int n, long ldc) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= m) return;
  for (int j = blockIdx.y; j < n; j += gridDim.y) C[(long)j * ldc + i] = 0.0;
}

}  // namespace

constexpr long CRT_ONE_COLUMN = 1L << 23;

hipError_t launch_crt(const uint8_t* rt, int m, int n, int m_pad, int n_pad, const int32_t* e, const int32_t* f,
                      const CrtConsts& c, double* C, int ldc, hipStream_t st) {
  // each thread reads four bytes of a column of every plane: m_pad must hold
  // whole groups of four rows
  if (m < 1 || n < 1 || m_pad < m || n_pad < n || m_pad % 4 || ldc < m) return hipErrorInvalidValue;
  // two columns per thread (the second one's loads overlap the first's
  // arithmetic); outputs of at most CRT_ONE_COLUMN entries take one column
  // per thread, twice the blocks, for more loads in flight
  const bool one_col = (long)m * n <= CRT_ONE_COLUMN;
  dim3 grid((m + 1023) / 1024, std::min(one_col ? n : (n + 1) / 2, 65535));
  const long plane = (long)m_pad * n_pad;
  const int ng = (c.s + 3) / 4;
  if (ng < 1 || ng > 5) return hipErrorInvalidValue;
#define OZ_CRT_NG(LL, WW)                                                                                     \
  switch (ng) {                                                                                             \
    case 1: OZ_CRT_CASE(LL, WW, 1); break;                                                                  \
    case 2: OZ_CRT_CASE(LL, WW, 2); break;                                                                  \
    case 3: OZ_CRT_CASE(LL, WW, 3); break;                                                                  \
    case 4: OZ_CRT_CASE(LL, WW, 4); break;                                                                  \
    default: OZ_CRT_CASE(LL, WW, 5); break;                                                                 \
  }
#define OZ_CRT_CASE(LL, WW, GG)                                                                               \
  hipLaunchKernelGGL((crt_kernel<LL, WW, GG>), grid, dim3(256), 0, st, rt, m, n, m_pad, plane, e, f, c, C, (long)ldc)
  if (c.W == 40) {
    switch (c.L) {
      case 1: OZ_CRT_NG(1, true); break;
      case 2: OZ_CRT_NG(2, true); break;
      case 3: OZ_CRT_NG(3, true); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (c.L) {
      case 1: OZ_CRT_NG(1, false); break;
      case 2: OZ_CRT_NG(2, false); break;
      case 3: OZ_CRT_NG(3, false); break;
      case 4: OZ_CRT_NG(4, false); break;
      case 5: OZ_CRT_NG(5, false); break;
      default: return hipErrorInvalidValue;
    }
  }
#undef OZ_CRT_NG
#undef OZ_CRT_CASE
  return hipGetLastError();
}

hipError_t launch_fill_zero(double* C, int m, int n, int ldc, hipStream_t st) {
  hipLaunchKernelGGL(fill_zero_kernel, dim3((m + 255) / 256, std::min(n, 65535)), dim3(256), 0, st, C, m, n, (long)ldc);
  return hipGetLastError();
}

}  // namespace oz
