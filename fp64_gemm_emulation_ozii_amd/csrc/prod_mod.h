// Reduction of an exact int32 product entry to its non-negative residue,
// C''_t = C'_t mod m_t (Ozaki II notes §4; §7 step 3).  Header-only and
// usable from host code, so that the arithmetic can be checked on the CPU.
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

// v mod m in [0, m) for any int32 v and 2 <= m <= 256, with inv = RN(1/m).
// (2v + 1) / 2m = v/m + 1/(2m) has an odd numerator over an even
// denominator, so it lies at least 1/(2m) from every integer.  The computed
// fma(v, inv, inv/2) is within 2^-21/m + 2^-53/m + 2^-23 < 1/(2m) of it
// (|v| <= 2^31, |inv - 1/m| <= 2^-52/m, one rounding of a value below 2^30
// + 1), so its floor is floor(v/m) exactly and v - m floor(v/m) is exact.
__host__ __device__ __forceinline__ uint32_t mod_product(int32_t v, double m, double inv) {
  const double x = (double)v;
  const double q = __builtin_floor(__builtin_fma(x, inv, 0.5 * inv));
  return (uint32_t)__builtin_fma(-q, m, x);
}

// Biased form, for accumulators that start at -h instead of 0: acc = v - h
// with v the product entry.  For odd m, h = (m - 1)/2, so that
// (v - h)/m = floor(v/m) + (r - h)/m with r = v mod m, and |r - h|/m is at
// most 1/2 - 1/(2m).  Rounding (v - h)/m to the nearest integer therefore
// gives floor(v/m), with the same 1/(2m) margin as above; one fma against
// the magic number 1.5 2^52 + beta rounds it (its grid spacing is 1 between
// 2^52 and 2^53), and the low 32 bits of the result are floor(v/m) + beta.
// The residue is needed as a byte only, so the rest runs modulo 256:
// acc + (256 - m)(floor(v/m) + beta) = r - h - m beta (mod 256), and
// beta = -h m^-1 (mod 256) leaves r in the low byte.  The product uses the
// low 24 bits of each factor, which keeps it one 24-bit multiply-add.
// For m = 256 the bias is 0 and the multiplier 0: the low byte of v is r.
// Valid for m = 256 and odd 3 <= m <= 255, and every int32 acc.
struct ModBias {
  int32_t bias;   // the accumulators' start value, -h
  uint32_t negm;  // 256 - m, or 0 for m = 256
  double magic;   // 1.5 2^52 + beta
};

// Integer operations only (1.5 2^52 + beta is assembled from its bits), so
// that on the GPU a wave-uniform m keeps every field in scalar registers.
__host__ __device__ inline ModBias mod_bias(int m) {
  const uint32_t um = (uint32_t)m, h = m == 256 ? 0u : (um - 1u) >> 1;
  uint32_t x = um;     // m^-1 mod 8 for odd m (every odd m is its own inverse there)
  x *= 2u - um * x;    // mod 2^6
  x *= 2u - um * x;    // mod 2^12
  const uint32_t beta = ((256u - h) * x) & 255u;  // 0 for m = 256, as h = 0
  return ModBias{-(int32_t)h, 256u - um, __builtin_bit_cast(double, 0x4338000000000000ull | beta)};
}

// Low byte: (acc + h) mod m, for acc = v - h as above.  The upper bytes are
// not cleared.
__host__ __device__ __forceinline__ uint32_t mod_product_biased(int32_t acc, uint32_t negm, double inv,
                                                                double magic) {
  const double t = __builtin_fma((double)acc, inv, magic);
  const uint32_t lo = (uint32_t)__builtin_bit_cast(uint64_t, t);
  return (lo & 0xffffffu) * (negm & 0xffffffu) + (uint32_t)acc;
}

}  // namespace oz
