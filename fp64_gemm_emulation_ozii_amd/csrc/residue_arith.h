// Per-entry arithmetic of the residue kernels: the symmetric residue
// r = A' - m floor(A'/m + 1/2) of an exact integer A' held in a double, in
// [-floor(m/2), ceil(m/2) - 1] for odd and even m alike (Ozaki II notes §4,
// §6).  Header-only and usable from host code as well, so that the
// arithmetic can be checked on the CPU against exact integers.
//
// The quotient is q = floor(fma(v, RN(1/m), 1/2)).  The fma result is within
// 2^(b-52) 1.01 / m of v/m + 1/2 when |v| < 2^b.  For odd m, v/m + 1/2 =
// (2v + m) / 2m has an odd numerator, so it is at least 1/2m away from every
// integer, and for m = 256 every step is exact: for |v| < 2^50 the floor is
// therefore always the exact one and r = fma(-q, m, v) needs no correction.
//
// * |A'| < 2^50 (residue_narrow): v = A'.  With am = A' + 1.5 2^52 (exact),
//   fma(-q, m, am) = 1.5 2^52 + r exactly, and the low 32 bits of its
//   pattern are r in two's complement, so no conversion is needed.
// * |A'| < 2^78 (split_wide, then residue_wide per modulus): A' = a2 2^52 +
//   a1 2^26 + a0 with a2 = floor(A' 2^-52) and a0, a1 in [0, 2^26), all
//   exact (a2 = 0, and one split, while |A'| < 2^53); v = a2 (2^52 mod m) +
//   a1 (2^26 mod m) + a0 is an exact integer congruent to A' with
//   |v| < 2^35, so the uncorrected reduction of v is the residue.
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

// |A'| < 2^50, am = A' + 1.5 2^52: r in the low 32 bits (two's complement).
__host__ __device__ __forceinline__ uint32_t residue_narrow(double a, double am, double m, double inv) {
  const double qf = __builtin_floor(__builtin_fma(a, inv, 0.5));
  return (uint32_t)__builtin_bit_cast(uint64_t, __builtin_fma(-qf, m, am));
}

// |A'| < 2^78 (BIG) or < 2^53: a becomes a0, a1 and a2 the higher pieces
// (a2 is left untouched unless BIG).
template <bool BIG>
__host__ __device__ __forceinline__ void split_wide(double& a, double& a1, double& a2) {
  if (BIG) {
    a2 = __builtin_floor(a * 0x1p-52);
    a = __builtin_fma(a2, -0x1p52, a);  // in [0, 2^52)
  }
  a1 = __builtin_floor(a * 0x1p-26);
  a = __builtin_fma(a1, -0x1p26, a);  // a0, in [0, 2^26)
}

// The residue of a0 + a1 2^26 + a2 2^52 (a2 only if BIG), c26 = 2^26 mod m,
// c52 = 2^52 mod m.
template <bool BIG>
__host__ __device__ __forceinline__ int residue_wide(double a0, double a1, double a2, double c26, double c52,
                                                     double m, double inv) {
  double v = __builtin_fma(a1, c26, a0);
  if (BIG) v = __builtin_fma(a2, c52, v);
  const double qf = __builtin_floor(__builtin_fma(v, inv, 0.5));
  return (int)__builtin_fma(-qf, m, v);
}

}  // namespace oz
