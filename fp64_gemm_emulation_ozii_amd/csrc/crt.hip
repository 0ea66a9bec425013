// CRT reconstruction, range reduction and unscaling (one output per thread).
//
// Ozaki II notes §4: X = sum_t C''_t M_t y_t (mod M); §5: with 2 c_max < M
// the symmetric representative is the integer product A'B' itself;
// §7 steps 4-6: accumulate, reduce, unscale by D^-1 and E^-1.
//
// 1. S_l = sum_t r_t w_{t,l}, where w_{t,l} < 2^32 are the 32-bit limbs of
//    W_t = M_t y_t (a small device table, staged in LDS per block).  Each term is < 2^40 and there are at most 20, so every
//    partial sum is an integer below 2^45 and FP64 fused multiply-adds are
//    exact.
// 2. Carry-propagate the S_l into 32-bit limbs Z_0..Z_L of Z = sum_t r_t W_t.
// 3. Q = rint(Z / M) from a double estimate (Z < 20*255*M, so the estimate
//    is within 2^-38 of Z/M and Q is right or off by one); X = Z - Q M in
//    two's complement limbs; one exact comparison against M/2 fixes an
//    off-by-one Q, giving the unique X with |X| < M/2.
// 4. C_ij = X * 2^(e_i + f_j - 2k) rounded once to nearest-even from a
//    64-bit window of |X| plus a sticky bit, with the rounding position moved
//    up for subnormal results and +-Inf past the double range.
#include "oz_internal.h"

namespace oz {

namespace {

// Round |X| * 2^(E - 63) to the nearest double, where T holds the 64 leading
// bits of |X| (bit 63 set) and `sticky` tells whether any lower bit is set.
__device__ __forceinline__ double round_window(uint64_t T, bool sticky, int E) {
  if (E >= 1024) return __builtin_inf();
  const int keep = min(53, E + 1075);  // significant bits the result can hold
  if (keep <= 0) {
    if (keep == 0) {
      // value in [2^-1075, 2^-1074): above the tie -> smallest subnormal
      const bool above = ((T << 1) != 0) || sticky;
      return above ? 4.9406564584124654e-324 : 0.0;
    }
    return 0.0;
  }
  const int drop = 64 - keep;  // 11..63
  const uint64_t mant = T >> drop;
  const uint64_t rem = T & ((1ull << drop) - 1);
  const uint64_t halfv = 1ull << (drop - 1);
  const bool up = (rem > halfv) || (rem == halfv && (sticky || (mant & 1)));
  return __builtin_ldexp((double)(mant + (up ? 1 : 0)), E - keep + 1);
}

// X * 2^(ei + fj - 2k) rounded once, from the exact limb sums S[0..L-1] of
// Z = sum_t r_t W_t (steps 2-4 above).
template <int L>
__device__ __forceinline__ double reconstruct(const double* S, const CrtConsts& c, int scale) {
  // 2. carries -> Z[0..L]
  uint32_t Z[L + 1];
  uint64_t carry = 0;
#pragma unroll
  for (int l = 0; l < L; ++l) {
    const uint32_t hi = (uint32_t)(S[l] * 0x1p-32);
    const uint32_t lo = (uint32_t)(S[l] - (double)hi * 0x1p32);
    const uint64_t v = (uint64_t)lo + carry;
    Z[l] = (uint32_t)v;
    carry = (v >> 32) + hi;
  }
  Z[L] = (uint32_t)carry;

  // 3. X = Z - Q M, then exact fix-up into (-M/2, M/2)
  double zf = (double)Z[L] * __builtin_ldexp(1.0, 32 * L) + (double)Z[L - 1] * __builtin_ldexp(1.0, 32 * (L - 1));
  if (L >= 2) zf += (double)Z[L - 2] * __builtin_ldexp(1.0, 32 * (L - 2));
  const uint32_t Q = (uint32_t)__builtin_rint(zf * c.invM);
  uint32_t X[L + 1];
  {
    uint64_t pc = 0;     // carry of Q*M
    int64_t borrow = 0;  // 0 or -1
#pragma unroll
    for (int l = 0; l <= L; ++l) {
      const uint64_t pm = (uint64_t)Q * c.M[l] + pc;
      pc = pm >> 32;
      const int64_t d = (int64_t)Z[l] - (int64_t)(uint32_t)pm + borrow;
      X[l] = (uint32_t)d;
      borrow = d < 0 ? -1 : 0;
    }
  }
  const bool neg0 = (X[L] >> 31) != 0;
  {
    // D = X - M/2 (if X >= 0) or X + M/2 (if X < 0); fix when D has X's sign
    uint32_t Dtop = 0;
    int64_t cb = 0;
#pragma unroll
    for (int l = 0; l <= L; ++l) {
      const int64_t d = neg0 ? (int64_t)X[l] + (int64_t)c.half[l] + cb : (int64_t)X[l] - (int64_t)c.half[l] + cb;
      Dtop = (uint32_t)d;
      cb = d >> 32;  // arithmetic: carry 1, borrow -1, or 0
    }
    const bool dneg = (Dtop >> 31) != 0;
    // X >= 0 and X - M/2 >= 0 (never == 0): X -= M;  X < 0 and X + M/2 < 0: X += M
    const bool fix = neg0 ? dneg : !dneg;
    if (fix) {
      int64_t cc = 0;
#pragma unroll
      for (int l = 0; l <= L; ++l) {
        const int64_t d = neg0 ? (int64_t)X[l] + (int64_t)c.M[l] + cc : (int64_t)X[l] - (int64_t)c.M[l] + cc;
        X[l] = (uint32_t)d;
        cc = d >> 32;
      }
    }
  }
  const bool neg = (X[L] >> 31) != 0;
  if (neg) {  // magnitude
    uint64_t cc = 1;
#pragma unroll
    for (int l = 0; l <= L; ++l) {
      const uint64_t v = (uint64_t)(~X[l]) + cc;
      X[l] = (uint32_t)v;
      cc = v >> 32;
    }
  }

  // 4. normalise so that X[L] holds the leading nonzero limb, then round
  int h = L;
#pragma unroll
  for (int it = 0; it < L; ++it) {
    if (X[L] == 0) {
#pragma unroll
      for (int l = L; l > 0; --l) X[l] = X[l - 1];
      X[0] = 0;
      --h;
    }
  }
  if (X[L] == 0) return 0.0;
  const int lz = __clz(X[L]);
  const uint64_t hi64 = ((uint64_t)X[L] << 32) | (uint64_t)X[L - 1];
  const uint32_t lo32 = (L >= 2) ? X[L - 2] : 0u;
  uint64_t T = hi64;
  uint32_t rest = lo32;
  if (lz > 0) {
    T = (hi64 << lz) | (uint64_t)(lo32 >> (32 - lz));
    rest = lo32 << lz;
  }
  bool sticky = rest != 0;
#pragma unroll
  for (int l = 0; l + 3 <= L; ++l) sticky = sticky || (X[l] != 0);
  const int E = 32 * h + 31 - lz + scale;  // exponent of the leading bit of |X| 2^scale
  const double res = round_window(T, sticky, E);
  return neg ? -res : res;
}

// Thread = 4 consecutive rows of one output column: the product residues of
// each modulus come in as one 32-bit load (the planes are padded to whole
// tiles, so rows up to the padded height are always readable).  The limbs of
// W_t sit in LDS, read once per modulus for all four rows.
template <int L>
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
  for (int j = blockIdx.y; j < n; j += gridDim.y) {
    const int fj = f[j];
    const uint8_t* p = rt + (long)j * m_pad + i0;
    // residues of the four rows for every modulus (planes past s are never
    // read: their slot loads plane s - 1 and is zeroed, as is its weight)
    uint32_t rr[OZGEMM_S_MAX];
#pragma unroll
    for (int t = 0; t < OZGEMM_S_MAX; ++t) {
      const uint32_t v = *reinterpret_cast<const uint32_t*>(p + (long)min(t, s - 1) * plane);
      rr[t] = (t < s) ? v : 0u;
    }
    // 1. exact FP64 limb sums for the four rows, moduli in groups of four
    double S[4][L];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int l = 0; l < L; ++l) S[u][l] = 0.0;
#pragma unroll
    for (int tg = 0; tg < OZGEMM_S_MAX; tg += 4) {
      if (tg < s) {
#pragma unroll
        for (int t = tg; t < tg + 4; ++t) {
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
      }
    }
    double res[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      res[u] = reconstruct<L>(S[u], c, ei[u] + fj - 2 * c.k);
      if (ei[u] == OZGEMM_EXP_NONFINITE || fj == OZGEMM_EXP_NONFINITE) res[u] = __builtin_nan("");
    }
    double* out = C + (long)j * ldc + i0;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (i0 + u < m) out[u] = res[u];
  }
}

__global__ void fill_zero_kernel(double* C, int m, int n, long ldc) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= m) return;
  for (int j = blockIdx.y; j < n; j += gridDim.y) C[(long)j * ldc + i] = 0.0;
}

}  // namespace

hipError_t launch_crt(const uint8_t* rt, int m, int n, int m_pad, int n_pad, const int32_t* e, const int32_t* f,
                      const CrtConsts& c, double* C, int ldc, hipStream_t st) {
  dim3 grid((m + 1023) / 1024, std::min(n, 65535));
  const long plane = (long)m_pad * n_pad;
  switch (c.L) {
#define OZ_CRT_CASE(LL)                                                                                      \
  case LL:                                                                                                    \
    hipLaunchKernelGGL((crt_kernel<LL>), grid, dim3(256), 0, st, rt, m, n, m_pad, plane, e, f, c, C, (long)ldc); \
    break;
    OZ_CRT_CASE(1)
    OZ_CRT_CASE(2)
    OZ_CRT_CASE(3)
    OZ_CRT_CASE(4)
    OZ_CRT_CASE(5)
#undef OZ_CRT_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_fill_zero(double* C, int m, int n, int ldc, hipStream_t st) {
  hipLaunchKernelGGL(fill_zero_kernel, dim3((m + 255) / 256, std::min(n, 65535)), dim3(256), 0, st, C, m, n, (long)ldc);
  return hipGetLastError();
}

}  // namespace oz
