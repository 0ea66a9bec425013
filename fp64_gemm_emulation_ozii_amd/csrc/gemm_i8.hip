// Per-modulus exact int8 GEMM on gfx950 matrix cores, with the product
// re-reduction fused into the epilogue.
//
// Ozaki II notes §4: one product C'_t = A'_t B'_t per modulus and no cross
// terms; §6: int8 residues with int32 accumulation are exact while
// q < 2^17 (|dot| <= q 2^14 < 2^31); §7 step 3: C''_t = C'_t mod m_t;
// §15: the independent moduli are batched into one launch (grid z = t).
//
// Operands are the K-contiguous residue planes written by the residue step:
// A_t is m_pad x q_pad (row i at i*q_pad), B_t is n_pad x q_pad (column j of
// B at j*q_pad), so the product is A_t B_t^T.  A block computes a BM x BN
// output tile with four wavefronts (2 x 2), each owning (BM/2) x (BN/2)
// built from 16x16 int32 tiles of v_mfma_i32_16x16x64_i8.
//
// Per 64-wide K slice, lane l of an MFMA supplies 16 bytes of row (l mod 16)
// of A and the same 16 K positions of column (l mod 16) of B, taken from
// K chunk (l / 16).  Both operands use the same lane -> K mapping, so every
// K index pairs with itself and the sum over the slice is the dot product
// whatever order the hardware walks the bytes in.  The int32 result tile
// holds rows 4*(l/16) + r, r = 0..3, of column (l mod 16) in lane l.
//
// LDS: each tile row (BK bytes) is stored as 16-byte chunks whose position
// is XOR-permuted by a function of the row, so that the 16 consecutive rows
// an MFMA operand load touches fall in distinct bank groups.  Two buffers:
// the next K slice is fetched from HBM into registers while the current
// one feeds the matrix cores, then written to the other buffer.
#include "oz_internal.h"

namespace oz {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

template <int BK>
__device__ __forceinline__ int swz(int row) {
  if constexpr (BK == 64) return ((row >> 1) ^ (row >> 3)) & 3;
  else return ((row >> 1) ^ (row << 2)) & 7;
}

template <int BM, int BN, int BK>
__global__ __launch_bounds__(256) void gemm_i8_kernel(const int8_t* __restrict__ Ares,
                                                       const int8_t* __restrict__ Bres, int m_pad, int n_pad,
                                                       int q_pad, GemmConsts c, int32_t* __restrict__ Ct,
                                                       uint8_t* __restrict__ rt) {
  constexpr int CPR = BK / 16;                 // 16-byte chunks per tile row
  constexpr int A_CHUNKS = BM * CPR / 256;     // chunk loads per thread
  constexpr int B_CHUNKS = BN * CPR / 256;
  constexpr int WTM = BM / 2, WTN = BN / 2;    // wave tile
  constexpr int FM = WTM / 16, FN = WTN / 16;  // 16x16 MFMA tiles per wave
  static_assert(A_CHUNKS >= 1 && B_CHUNKS >= 1, "tile too small");

  __shared__ __attribute__((aligned(16))) int8_t As[2][BM * BK];
  __shared__ __attribute__((aligned(16))) int8_t Bs[2][BN * BK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int t = blockIdx.z;
  const int m0 = blockIdx.y * BM;
  const int n0 = blockIdx.x * BN;

  const int8_t* Ag = Ares + (long)t * m_pad * q_pad + (long)m0 * q_pad;
  const int8_t* Bg = Bres + (long)t * n_pad * q_pad + (long)n0 * q_pad;

  // global -> register chunk coordinates (fixed per thread)
  int a_off[A_CHUNKS], a_lds[A_CHUNKS], b_off[B_CHUNKS], b_lds[B_CHUNKS];
#pragma unroll
  for (int p = 0; p < A_CHUNKS; ++p) {
    const int cidx = tid + 256 * p;
    const int row = cidx / CPR, kc = cidx % CPR;
    a_off[p] = row * q_pad + kc * 16;
    a_lds[p] = row * BK + ((kc ^ swz<BK>(row)) * 16);
  }
#pragma unroll
  for (int p = 0; p < B_CHUNKS; ++p) {
    const int cidx = tid + 256 * p;
    const int row = cidx / CPR, kc = cidx % CPR;
    b_off[p] = row * q_pad + kc * 16;
    b_lds[p] = row * BK + ((kc ^ swz<BK>(row)) * 16);
  }

  uint4 ra[A_CHUNKS], rb[B_CHUNKS];
#pragma unroll
  for (int p = 0; p < A_CHUNKS; ++p) ra[p] = *reinterpret_cast<const uint4*>(Ag + a_off[p]);
#pragma unroll
  for (int p = 0; p < B_CHUNKS; ++p) rb[p] = *reinterpret_cast<const uint4*>(Bg + b_off[p]);
#pragma unroll
  for (int p = 0; p < A_CHUNKS; ++p) *reinterpret_cast<uint4*>(&As[0][a_lds[p]]) = ra[p];
#pragma unroll
  for (int p = 0; p < B_CHUNKS; ++p) *reinterpret_cast<uint4*>(&Bs[0][b_lds[p]]) = rb[p];
  __syncthreads();

  v4i acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = v4i{0, 0, 0, 0};

  const int nk = q_pad / BK;
  const int lrow = lane & 15;
  const int lkc = lane >> 4;  // 0..3: K chunk within a 64-wide slice

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    // prefetch the next slice (the last iteration re-reads its own slice
    // into the idle buffer, which keeps the loop free of branches)
    const int kn = min(kt + 1, nk - 1) * BK;
#pragma unroll
    for (int p = 0; p < A_CHUNKS; ++p) ra[p] = *reinterpret_cast<const uint4*>(Ag + a_off[p] + kn);
#pragma unroll
    for (int p = 0; p < B_CHUNKS; ++p) rb[p] = *reinterpret_cast<const uint4*>(Bg + b_off[p] + kn);
#pragma unroll
    for (int ks = 0; ks < BK / 64; ++ks) {
      v4i af[FM], bf[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int row = wm * WTM + i * 16 + lrow;
        const int kc = ks * 4 + lkc;
        af[i] = *reinterpret_cast<const v4i*>(&As[cur][row * BK + ((kc ^ swz<BK>(row)) * 16)]);
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int row = wn * WTN + j * 16 + lrow;
        const int kc = ks * 4 + lkc;
        bf[j] = *reinterpret_cast<const v4i*>(&Bs[cur][row * BK + ((kc ^ swz<BK>(row)) * 16)]);
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
#pragma unroll
    for (int p = 0; p < A_CHUNKS; ++p) *reinterpret_cast<uint4*>(&As[cur ^ 1][a_lds[p]]) = ra[p];
#pragma unroll
    for (int p = 0; p < B_CHUNKS; ++p) *reinterpret_cast<uint4*>(&Bs[cur ^ 1][b_lds[p]]) = rb[p];
    __syncthreads();
  }

  // ---- epilogue: int32 planes and/or residues mod m_t ----
  const long plane = (long)m_pad * n_pad;
  // select this plane's modulus without indexing the by-value argument
  // dynamically (which would copy it to scratch)
  int mt = c.m[0];
  double inv = c.inv[0];
#pragma unroll
  for (int u = 1; u < OZGEMM_S_MAX; ++u) {
    mt = (u == t) ? c.m[u] : mt;
    inv = (u == t) ? c.inv[u] : inv;
  }
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int row = m0 + wm * WTM + i * 16 + 4 * (lane >> 4);
      const int col = n0 + wn * WTN + j * 16 + (lane & 15);
      const long off = (long)t * plane + (long)col * m_pad + row;
      const v4i v = acc[i][j];
      if (Ct != nullptr) *reinterpret_cast<v4i*>(Ct + off) = v;
      if (rt != nullptr) {
        uint32_t packed = 0;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const double d = (double)v[r];
          const double qf = __builtin_floor(d * inv);
          int ri = (int)__builtin_fma(-qf, (double)mt, d);
          ri = ri < 0 ? ri + mt : ri;
          ri = ri >= mt ? ri - mt : ri;
          packed |= (uint32_t)ri << (8 * r);
        }
        *reinterpret_cast<uint32_t*>(rt + off) = packed;
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm(const int8_t* Ares, const int8_t* Bres, int m_pad, int n_pad, int q_pad, const GemmConsts& c,
                       int32_t* Ct, uint8_t* rt, hipStream_t st) {
  constexpr int BM = 128, BN = 128, BK = 64;
  if (m_pad % BM || n_pad % BN || q_pad % BK) return hipErrorInvalidValue;
  dim3 grid(n_pad / BN, m_pad / BM, c.s);
  hipLaunchKernelGGL((gemm_i8_kernel<BM, BN, BK>), grid, dim3(256), 0, st, Ares, Bres, m_pad, n_pad, q_pad, c, Ct,
                     rt);
  return hipGetLastError();
}

}  // namespace oz
