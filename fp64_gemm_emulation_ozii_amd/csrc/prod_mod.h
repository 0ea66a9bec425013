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

}  // namespace oz
