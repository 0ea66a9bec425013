// Sustained rate of the int8 matrix cores, for measurement: a register-only
// loop of v_mfma_i32_16x16x64_i8 in the operand order of the product
// kernel (each A fragment meets every B fragment in turn), with 4 x 8 tiles
// of 16 x 16 per wavefront (32 independent accumulators, 128 accumulator
// words per lane) on pseudo-random operands.  Under the part's power limit
// the rate such a loop sustains, not the clock-rate figure, is the ceiling
// the product kernel can approach; the benchmark reports the product against
// both.
//
// Operands: word w of wavefront g is lowbias32(w + seed * 0x9e3779b9),
// Wellons' 32-bit integer hash, with w = ((g * 12 + f) * 64 + lane) * 4 + r
// for fragment f (0..3 the A rows of tile row f, 4..11 the B columns of tile
// column f - 4) and word r of the lane's 16 bytes.
#include "oz_internal.h"

namespace oz {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t lowbias32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

// Each wavefront runs `steps` steps of 32 MFMAs and writes the XOR of all
// its accumulator words to sink[global wavefront index].
__global__ __launch_bounds__(256, 1) void mfma_ceiling_kernel(int steps, uint32_t seed, uint32_t* __restrict__ sink) {
  constexpr int FA = 4, FB = 8;
  const int lane = threadIdx.x & 63;
  const uint32_t g = blockIdx.x * 4u + (threadIdx.x >> 6);
  const uint32_t base = seed * 0x9e3779b9u;
  v4i a[FA], b[FB];
#pragma unroll
  for (int f = 0; f < FA + FB; ++f) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int x = (int)lowbias32(((g * (FA + FB) + f) * 64u + lane) * 4u + r + base);
      if (f < FA)
        a[f][r] = x;
      else
        b[f - FA][r] = x;
    }
  }
  v4i acc[FA][FB];
#pragma unroll
  for (int i = 0; i < FA; ++i)
#pragma unroll
    for (int j = 0; j < FB; ++j) acc[i][j] = v4i{0, 0, 0, 0};
  for (int it = 0; it < steps; ++it) {
#pragma unroll
    for (int i = 0; i < FA; ++i)
#pragma unroll
      for (int j = 0; j < FB; ++j) {
        acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[i], b[j], acc[i][j], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);  // the product kernel's issue order
      }
  }
  uint32_t x = 0;
#pragma unroll
  for (int i = 0; i < FA; ++i)
#pragma unroll
    for (int j = 0; j < FB; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) x ^= (uint32_t)acc[i][j][r];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x ^= (uint32_t)__shfl_xor((int)x, o, 64);
  if (lane == 0) sink[g] = x;
}

}  // namespace

hipError_t launch_mfma_ceiling(int blocks, int steps, uint32_t seed, uint32_t* sink, hipStream_t st) {
  hipLaunchKernelGGL(mfma_ceiling_kernel, dim3(blocks), dim3(256), 0, st, steps, seed, sink);
  return hipGetLastError();
}

}  // namespace oz
