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
//
// reconstruct40 is the same computation on 40-bit limbs (used while
// log2 M <= 120, i.e. at most three limbs): S[l] = sum_t r_t w_{t,l} with
// w_{t,l} < 2^40 stays below 2^53 for s <= 15, the balanced carries leave
// limbs in [-2^39, 2^39], and the single rounding of X = x0 + x1 2^40 +
// x2 2^80 is done in FP64 as the correctly rounded sum of three exact terms
// (Boldo and Melquiond, "Emulation of FMA and correctly rounded sums:
// proved algorithms using rounding to odd", IEEE TC 2008: two error-free
// additions, a round-to-odd addition of the two errors, and one final
// round-to-nearest addition).  Results that would be subnormal take an
// exact 128-bit integer path instead, since scaling a rounded value into the
// subnormal range would round twice.
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


// ---------------------------------------------------------------------------
// 40-bit limbs
// ---------------------------------------------------------------------------

// Balanced carries between 40-bit limbs: each limb but the top one ends in
// [-2^39, 2^39].  Exact while every limb stays below 2^53.
template <int L>
__host__ __device__ __forceinline__ void carry40(double* x) {
#pragma unroll
  for (int l = 0; l + 1 < L; ++l) {
    const double c = __builtin_rint(x[l] * 0x1p-40);
    x[l] = __builtin_fma(c, -0x1p40, x[l]);
    x[l + 1] += c;
  }
}

// s = a + b rounded to odd: the exact sum when representable, otherwise
// whichever neighbour of it has an odd last significand bit.
__host__ __device__ __forceinline__ double add_round_odd(double a, double b) {
  const double s = a + b;
  const double bb = s - a;
  const double e = (a - (s - bb)) + (b - bb);  // a + b = s + e exactly
  uint64_t u = __builtin_bit_cast(uint64_t, s);
  if (e != 0.0 && (u & 1u) == 0) {
    // away from zero when e has the sign of s, towards zero otherwise
    const bool away = (e > 0.0) == (s > 0.0);
    u = away ? u + 1 : u - 1;
  }
  return __builtin_bit_cast(double, u);
}

// Exact rounding of X 2^scale, X = x0 + x1 2^40 + x2 2^80 (limbs exact,
// |x_l| < 2^53), from the 128-bit integer X; used for subnormal results.
__host__ __device__ inline double round_limbs40_exact(double x0, double x1, double x2, int scale) {
  const __int128 X = (__int128)(int64_t)x0 + (__int128)(int64_t)x1 * ((__int128)1 << 40) +
                     (__int128)(int64_t)x2 * ((__int128)1 << 80);
  if (X == 0) return 0.0;
  const bool neg = X < 0;
  const unsigned __int128 u = neg ? (unsigned __int128)(-X) : (unsigned __int128)X;
  const uint64_t hi = (uint64_t)(u >> 64), lo = (uint64_t)u;
  const int top = hi ? 127 - __builtin_clzll(hi) : 63 - __builtin_clzll(lo);  // leading bit position
  uint64_t T;
  bool sticky;
  if (top >= 63) {
    const int sh = top - 63;
    T = (uint64_t)(u >> sh);
    sticky = sh > 0 && (u & (((unsigned __int128)1 << sh) - 1)) != 0;
  } else {
    T = lo << (63 - top);
    sticky = false;
  }
  const double r = round_window(T, sticky, top + scale);
  return neg ? -r : r;
}

template <int L>
__host__ __device__ __forceinline__ double reconstruct40(const double* S_in, const CrtModulus& K, int scale) {
  static_assert(L >= 1 && L <= 3, "40-bit limbs: at most three");
  // 2. X = Z - Q M (|S_l| < 2^53 - 2^52, Q M_l < 2^52: exact)
  double zf = S_in[L - 1] * __builtin_ldexp(1.0, 40 * (L - 1));
  if (L >= 2) zf = __builtin_fma(S_in[L - 2], __builtin_ldexp(1.0, 40 * (L - 2)), zf);
  const double Q = __builtin_rint(zf * K.invM);
  double x[L];
#pragma unroll
  for (int l = 0; l < L; ++l) x[l] = __builtin_fma(-Q, K.Ml[l], S_in[l]);
  carry40<L>(x);

  // 3. symmetric representative
  double xa = x[0];
  if (L >= 2) xa = __builtin_fma(x[1], 0x1p40, xa);
  if (L >= 3) xa = __builtin_fma(x[2], 0x1p80, xa);
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
    carry40<L>(d);
    if (sign_limbs<L>(d) == sx) shift_m = sx;
  }
  if (shift_m != 0) {
#pragma unroll
    for (int l = 0; l < L; ++l) x[l] = __builtin_fma(-(double)shift_m, K.Ml[l], x[l]);
    carry40<L>(x);
  }

  // 4. z = RN(X): x0, x1 2^40 and x2 2^80 are exact; with the balanced
  //    limbs |x0| < 2^40 <= |x1 2^40| and |x1 2^40 + x0| < 2^80 <= |x2 2^80|
  //    (when nonzero), so both error-free additions may be Fast2Sum
  double z;
  if (L == 1) {
    z = x[0];
  } else if (L == 2) {
    z = __builtin_fma(x[1], 0x1p40, x[0]);
  } else {
    const double b = x[1] * 0x1p40, c = x[0], a = x[L - 1] * 0x1p80;
    const double uh = b + c, ul = c - (uh - b);
    const double th = a + uh, tl = uh - (th - a);
    z = th + add_round_odd(tl, ul);
  }
  if (z == 0.0) return 0.0;
  const int ez = (int)((__builtin_bit_cast(uint64_t, z) >> 52) & 0x7ff) - 1023;  // z is an integer, normal
  if (ez + scale < -1022) return round_limbs40_exact(x[0], L >= 2 ? x[1] : 0.0, L >= 3 ? x[2] : 0.0, scale);
  return __builtin_ldexp(z, scale);
}

}  // namespace oz
