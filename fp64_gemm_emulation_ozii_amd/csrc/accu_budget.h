// The exact budget comparison of OS II-accu (Ozaki II notes §9), shared by
// the combine kernel and a host test.  An entry whose two-band bound is
// N / (127^2 2^14) admits row and column bit counts with
// 2^(a_i + b_j) N / (127^2 2^14) <= M/2 - 1, i.e. a_i + b_j <=
// floor(log2(V / N)) with V = (M/2 - 1) 127^2 2^14.
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

// floor(log2(V / N)) for 0 < N < 2^62 and a V of bv >= 64 bits whose top 64
// bits are vtop: with bn the bit length of N and t0 = bv - bn, N 2^t0 <= V
// exactly when N <= floor(V / 2^t0) = vtop >> (64 - bn) (the floors of
// divisions by powers of two compose), and then t0 is the answer (N 2^(t0+1)
// >= 2^bv > V); otherwise t0 - 1 is (N 2^(t0-1) < 2^(bv-1) <= V).
__host__ __device__ __forceinline__ int floor_log2_ratio(uint64_t N, uint64_t vtop, int bv) {
  const int bn = 64 - __builtin_clzll(N);
  const int t0 = bv - bn;
  return N <= (vtop >> (64 - bn)) ? t0 : t0 - 1;
}

}  // namespace oz
