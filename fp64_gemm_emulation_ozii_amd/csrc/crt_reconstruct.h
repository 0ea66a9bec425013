// Exact CRT reconstruction, range reduction and single rounding of one
// output, from the limb sums of Z = sum_t r_t W_t (Ozaki II notes §4, §5,
// §7 steps 4-6).  Header-only and usable from host code as well, so that the
// arithmetic can be checked on the CPU against exact integers.
//
// Input: S[0..L-1], S[l] = sum_t r_t w_{t,l} with w_{t,l} the 32-bit limbs
// of W_t = M_t y_t; every S[l] is an integer below 2^46, held exactly in a
// double.  Z = sum_l S[l] 2^(32 l).
//
// 1. Q = rint(Z / M) from the two top limb sums; Q <= 20 * 255, right or off
//    by one.  X[l] = S[l] - Q M[l] is exact (|.| < 2^47).
// 2. Balanced carries: c = floor(X[l] 2^-32 + 1/2) moves into X[l+1], leaving
//    X[l] in [-2^31, 2^31).  All operations are exact in FP64.
// 3. With balanced limbs the sign of X is the sign of its top nonzero limb
//    (the lower ones add up to less than one unit of it).  |X| is compared
//    with M/2 on a double approximation; only inside a band of relative width
//    2^-40 around M/2 is the comparison made exactly on the limbs.  Outside
//    (-M/2, M/2) X moves by one M, exactly.
// 4. X in two's-complement 64-bit words, |X|, then rounding to nearest-even
//    of |X| 2^scale from a 64-bit window plus a sticky bit; the rounding
//    position moves up for subnormal results, and results past the double
//    range become +-Inf.
#pragma once

#include <stdint.h>

#ifndef __HIPCC__
#ifndef __host__
#define __host__
#endif
#ifndef __device__
#define __device__
#endif
#ifndef __forceinline__
#define __forceinline__ inline
#endif
#endif

namespace oz {

// |X| 2^(E - 63) rounded to the nearest double, where T holds the 64 leading
// bits of |X| (bit 63 set) and `sticky` tells whether any lower bit is set.
__host__ __device__ __forceinline__ double round_window(uint64_t T, bool sticky, int E) {
  if (E >= 1024) return __builtin_inf();
  if (E >= -1022) {
    // normal result: 53 significant bits; the rounded significand (bit 52
    // set, or 2^53 after a carry) added to the exponent field gives the
    // double directly, including the carry into the next binade and the
    // overflow to +Inf at E = 1023
    const uint64_t mant = T >> 11;
    const uint64_t rem = T & 0x7ff;
    const bool up = (rem > 0x400) || (rem == 0x400 && (sticky || (mant & 1)));
    return __builtin_bit_cast(double, ((uint64_t)(E + 1022) << 52) + mant + (up ? 1 : 0));
  }
  const int keep = E + 1075;  // significant bits a subnormal result can hold (< 53)
  if (keep <= 0) {
    if (keep == 0) {
      // value in [2^-1075, 2^-1074): above the tie -> smallest subnormal
      const bool above = ((T << 1) != 0) || sticky;
      return above ? 4.9406564584124654e-324 : 0.0;
    }
    return 0.0;
  }
  const int drop = 64 - keep;  // 12..63
  const uint64_t mant = T >> drop;
  const uint64_t rem = T & ((1ull << drop) - 1);
  const uint64_t halfv = 1ull << (drop - 1);
  const bool up = (rem > halfv) || (rem == halfv && (sticky || (mant & 1)));
  return __builtin_ldexp((double)(mant + (up ? 1 : 0)), E - keep + 1);
}

// Move floor(x[l] 2^-32 + 1/2) (or floor(x[l] 2^-32) when NONNEG) from each
// limb into the next one.
template <int L, bool NONNEG>
__host__ __device__ __forceinline__ void carry_limbs(double* x) {
#pragma unroll
  for (int l = 0; l + 1 < L; ++l) {
    const double c = NONNEG ? __builtin_floor(x[l] * 0x1p-32) : __builtin_floor(x[l] * 0x1p-32 + 0.5);
    x[l] = __builtin_fma(c, -0x1p32, x[l]);
    x[l + 1] += c;
  }
}

// Sign (-1, 0, +1) of sum_l x[l] 2^(32 l) for balanced limbs.
template <int L>
__host__ __device__ __forceinline__ int sign_limbs(const double* x) {
  int sg = 0;
#pragma unroll
  for (int l = 0; l < L; ++l) sg = (x[l] > 0.0) ? 1 : (x[l] < 0.0) ? -1 : sg;
  return sg;
}

// Constants of M: limbs (as doubles), limbs of M/2 (M is even), M/2 and 1/M.
struct CrtModulus {
  double Ml[5];
  double Hl[5];
  double halfM;
  double invM;
};

template <int L>
__host__ __device__ __forceinline__ double reconstruct_limbs(const double* S_in, const CrtModulus& K, int scale) {
  // 2. X = Z - Q M, limb by limb on the raw sums (|S_l| < 2^46 and
  //    Q M_l < 2^45, so every limb stays an exact integer below 2^47)
  double zf = S_in[L - 1] * __builtin_ldexp(1.0, 32 * (L - 1));
  if (L >= 2) zf += S_in[L - 2] * __builtin_ldexp(1.0, 32 * (L - 2));
  const double Q = __builtin_rint(zf * K.invM);
  double x[L];
#pragma unroll
  for (int l = 0; l < L; ++l) x[l] = __builtin_fma(-Q, K.Ml[l], S_in[l]);
  carry_limbs<L, false>(x);

  // 3. symmetric representative
  double xa = x[L - 1] * __builtin_ldexp(1.0, 32 * (L - 1));
  if (L >= 2) xa += x[L - 2] * __builtin_ldexp(1.0, 32 * (L - 2));
  if (L >= 3) xa += x[L - 3] * __builtin_ldexp(1.0, 32 * (L - 3));
  const double ax = xa < 0 ? -xa : xa;
  int shift_m = 0;  // X -> X - shift_m * M
  if (ax > K.halfM * (1.0 + 0x1p-40)) {
    shift_m = xa > 0 ? 1 : -1;
  } else if (ax >= K.halfM * (1.0 - 0x1p-40)) {
    // exact: is |X| > M/2 ?  (|X| = M/2 cannot occur)
    const int sx = sign_limbs<L>(x);
    double d[L];
#pragma unroll
    for (int l = 0; l < L; ++l) d[l] = x[l] - (double)sx * K.Hl[l];
    carry_limbs<L, false>(d);
    if (sign_limbs<L>(d) == sx) shift_m = sx;
  }
  if (shift_m != 0) {
#pragma unroll
    for (int l = 0; l < L; ++l) x[l] = __builtin_fma(-(double)shift_m, K.Ml[l], x[l]);
    carry_limbs<L, false>(x);
  }

  // 4. X as a two's-complement integer in 64-bit words (each balanced limb
  //    fits int32: |X| < M/2 < 2^(32 L - 1) keeps even the top limb below
  //    2^31), then |X| and one rounding from its 64 leading bits.
  constexpr int NW = (L + 1) / 2;
  uint64_t w[NW];
#pragma unroll
  for (int v = 0; v < NW; ++v) {
    const int64_t lo = (int64_t)(int32_t)x[2 * v];
    const int64_t hi = (2 * v + 1 < L) ? (int64_t)(int32_t)x[2 * v + 1] : 0;
    w[v] = (uint64_t)lo + ((uint64_t)hi << 32);
  }
  // word v holds lo + hi 2^32 as a signed value; carry the signs upward
#pragma unroll
  for (int v = 0; v + 1 < NW; ++v) {
    const int64_t sv = (int64_t)w[v];  // signed value of this word (fits: |.| < 2^63)
    if (sv < 0) w[v + 1] -= 1;         // w[v] read as unsigned = sv + 2^64
  }
  // |X|: two's-complement negation under a mask (no branch)
  const uint64_t negmask = (uint64_t)((int64_t)w[NW - 1] >> 63);
  uint64_t carry = negmask & 1u;
#pragma unroll
  for (int v = 0; v < NW; ++v) {
    const uint64_t nv = (w[v] ^ negmask) + carry;
    carry = (carry != 0 && nv == 0) ? 1u : 0u;
    w[v] = nv;
  }
  // leading 64 bits: top word with nonzero content, and the next one
  int top = -1;
#pragma unroll
  for (int v = 0; v < NW; ++v)
    if (w[v] != 0) top = v;
  if (top < 0) return 0.0;
  uint64_t hiw = 0, low = 0, rest = 0;
#pragma unroll
  for (int v = 0; v < NW; ++v) {
    if (v == top) hiw = w[v];
    if (v == top - 1) low = w[v];
    if (v < top - 1) rest |= w[v];
  }
  const int lz = __builtin_clzll(hiw);
  const uint64_t T = lz ? (hiw << lz) | (low >> (64 - lz)) : hiw;
  const bool sticky = ((lz ? (low << lz) : low) != 0) || rest != 0;
  // the leading bit of |X| is bit 64 top + 63 - lz; T holds it in bit 63
  const double res = round_window(T, sticky, 64 * top + 63 - lz + scale);
  return __builtin_bit_cast(double, __builtin_bit_cast(uint64_t, res) | (negmask << 63));
}

}  // namespace oz
