// Exact int8 GEMMs on gfx950 matrix cores: one per modulus for Scheme II
// (with the product re-reduction fused into the epilogue), and the slice
// products of the Scheme I path.
//
// Ozaki II notes §4: one product C'_t = A'_t B'_t per modulus and no cross
// terms; §6: int8 residues with int32 accumulation are exact while
// q < 2^17 (|dot| <= q 2^14 < 2^31); §7 step 3: C''_t = C'_t mod m_t;
// §15: the independent moduli are batched into one launch.  Ozaki I notes
// (INT matrix multiplication algorithm, group-wise accumulation): slice
// products A_s B_t, optionally several with the same s + t summed into one
// int32 accumulator.
//
// Operands are K-contiguous int8 planes: A_t is m_pad x q_pad (row i at
// i*q_pad), B_t is n_pad x q_pad (column j of B at j*q_pad), so each product
// is A_t B_t^T.  A block computes a 256 x 256 output tile from 16x16 int32
// tiles of v_mfma_i32_16x16x64_i8, with four wavefronts (2 x 2, one per
// SIMD, 128 x 128 each: residue-only products that walk many K slices) or
// eight (2 x 4, two per SIMD, 128 x 64 each: residue-only products that
// walk few, and every int32-output form).  In the multi-product (plan) form
// an output plane is the sum of `count` products (A_{a0+u}, B_{b0-u}),
// u = 0..count-1, walked as one long K loop.
//
// LDS: each tile row (BK bytes) is stored as 16-byte chunks whose position
// is XOR-permuted by a function of the row, so that the rows an MFMA operand
// load touches fall in distinct bank groups.  K slices move from HBM straight
// into LDS through two buffers.
//
// Grids (gemm_grid.h): a block's linear id picks its plane and tile; skinny
// products with a long inner dimension are cut into K parts whose residues a
// small kernel adds mod m_t; residue-only launches with more blocks than
// compute units run as one persistent block per unit that walks the tiles
// the hardware would have handed it, loading the next tile's first slice
// while the finished one is reduced and written.
#include "oz_internal.h"
#include "prod_mod.h"

namespace oz {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

// Physical 16-byte chunk of logical chunk kc in tile row `row` is kc ^ swz(row).
// A wavefront's 16-byte LDS reads are served 16 lanes at a time from 64
// four-byte banks (256 bytes); an MFMA operand load sends 16 consecutive tile
// rows to one group, so the 16 chunks must land in 16 different 16-byte bank
// slots.  With 128-byte rows the slot is 8 (row & 1) + physical chunk, and
// ((row >> 1) ^ (row << 2)) & 7 takes 8 distinct values on the even and on
// the odd rows of every 16-row window (it also keeps 8-row groups distinct).
// It depends on row mod 16 only, so a lane's source offset for the direct
// LDS loads takes one of two values (even / odd 1 KB block).
template <int BK>
__host__ __device__ __forceinline__ int swz(int row) {
  static_assert(BK == 128, "the swizzle is laid out for 128-byte rows");
  return ((row >> 1) ^ (row << 2)) & 7;  // always < 8: stays inside the row
}

// s_waitcnt with only the vector-memory counter constrained to <= N.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// An accumulator entry read out of its AGPR.  The "a" constraint keeps the
// 256 accumulators of the main kernel in AGPRs up to the epilogue; read as
// plain values, each used twice by the biased reduction, the compiler moved
// some of them into VGPRs and spilled other values.
__device__ __forceinline__ int32_t from_agpr(int32_t x) {
  int32_t r;
  asm("v_accvgpr_read_b32 %0, %1" : "=v"(r) : "a"(x));
  return r;
}

// The low bytes of four words as one word, first word lowest.
__device__ __forceinline__ uint32_t low_bytes(uint32_t b0, uint32_t b1, uint32_t b2, uint32_t b3) {
  const uint32_t lo = __builtin_amdgcn_perm(b1, b0, 0x0c0c0400u);  // b0.0, b1.0, 0, 0
  const uint32_t hi = __builtin_amdgcn_perm(b3, b2, 0x0c0c0400u);  // b2.0, b3.0, 0, 0
  return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

// BM x BN output tile per block of WM x WN wavefronts; each wavefront owns a
// (BM/WM) x (BN/WN) sub-tile of MT x MT = 16 x 16 tiles of
// v_mfma_i32_16x16x64_i8.  On random int8 operands the chip's power limit
// lets this instruction sustain about 15% more operations per second than
// v_mfma_i32_32x32x32_i8 (3.65 against 3.15 POP/s in a register-only loop);
// the 8192^3 product phase runs 4-5% faster with it.  The int32-output
// forms used 32 x 32 tiles while they ran four wavefronts, whose 256
// accumulators went to scratch with 16-wide tiles; with eight wavefronts
// the 128 accumulators fit in registers, and Scheme I at 4096^3, k = 8,
// runs 1% (RN) and 8% (Hybrid) faster.  Lane l supplies 16 bytes of row
// (l mod 16) of A (column (l mod 16) of B) from K chunk l / 16 of the
// 64-wide K step and receives rows 4 (l / 16) + r, r = 0..3, of column
// (l mod 16).  Both operands use the same lane -> K mapping, so the product
// is the dot product over the step whatever order the hardware takes the
// bytes in.
//
// Data movement and instruction order:
//  * K slices of BK bytes go from HBM straight into LDS (global_load_lds, 16
//    bytes per lane, no register staging) through two buffers.
//  * One barrier per slice, placed before the last K step's MFMAs: it
//    publishes slice kt + 1 (this wave's loads of it have landed) and retires
//    buffer kt mod 2 (this wave's reads of it are in registers).
//  * Every step is a fixed sequence of MFMA slots (64 with four
//    wavefronts).  The fragments of the next step are read from LDS, one
//    after every RS-th slot, and the 16 loads of the slice two ahead go
//    after slots 1, 1 + RS, 1 + 2 RS, ... of the window that follows the
//    barrier (the last step of slice kt, then the next slice's steps): over
//    its first 1024 MFMA cycles.
//    Spreading the loads this way keeps their issue from stalling the MFMA
//    stream, and the last of them still has half a slice to land.
//    (Measured at 8192^3 x 14 planes: 7.1 ms with the loads issued as one
//    burst per slice, 6.3 ms with this order.)
//  * Eight wavefronts (WM x WN = 2 x 4, 128 x 64 each, two per SIMD, 128
//    accumulators): 32 MFMA slots and 12 fragment reads per step, which do
//    not divide evenly.  A fragment i is re-read right after its last MFMA
//    (slot 4 i + 3), so its old and new values can share registers, B
//    fragment j after slot 8 j + 1, and the 8 loads per slice go after slots
//    2, 6, ..., 30.  Each wavefront reads 1.5x the LDS bytes per MFMA, but
//    one wavefront's waits, barrier arrival and epilogue run beside the
//    other's MFMAs.  Same-box A/B against four wavefronts (s = 14): 3-5%
//    faster at 16384^2 x 1024, 2.2% at 16384^2 x 2048, 1.3-1.4% at 1024^3
//    and 2048^3 (8 and 16 K slices per block); 1.3-1.7% slower at
//    8192^2 x 4096 and 16384^3, within +-2% at 8192^3 (32-128 slices).  At
//    K <= 512 it also beats a kernel of two 256 x 128 blocks per CU (6-10%
//    at K = 512), whose smaller tile loads 1.5x the bytes per MAC.
// K parts (gemm_grid.h): plane index p s + t of a residue-only launch is
// part p of modulus t, covering K slices [k_begin + p k_slices, + k_slices)
// clipped to q_pad; it writes its residue to plane p s + t of rt.  With one
// part the plane index is the modulus.
// Inner dimension q >= 2^17 whose parts do not fit (Ozaki II notes §6, block
// products): one launch per K block of at most KBLOCK_K entries, each exact
// in int32 (|.| <= 2^16 2^14 < 2^31); with ACC_RT the epilogue adds the
// block's residue to the residue already in rt, mod m_t.
constexpr int KBLOCK_K = 1 << 16;

// Slot plan of one K step (see above): fragment f of the next step is read
// after MFMA slot read_slot, load li of a slice after slot load_slot of its
// window.  Four wavefronts: rs = slots / fragments.  Eight: fn B fragments
// (f < fn), then the A fragments.
constexpr int read_slot(bool eight, int rs, int fn, int f) {
  return eight ? (f < fn ? 8 * f + 1 : fn * (f - fn) + fn - 1) : rs * f;
}
constexpr int load_slot(bool eight, int rs, int li) { return eight ? 4 * li + 2 : rs * li + 1; }
// loads of a slice that fall in the last step of the slice before it
constexpr int early_loads(bool eight, int rs, int lpw, int slots) {
  int h = 0;
  for (int li = 0; li < lpw; ++li) h += load_slot(eight, rs, li) < slots;
  return h;
}

// Residue-only launches whose blocks walk at most this many K slices use
// eight wavefronts per block.
constexpr int EIGHT_WAVE_MAX_SLICES = 16;

template <int BM, int BN, int BK, int WM, int WN, bool WRITE_CT, bool WRITE_RT, bool MULTI, bool ACC_RT = false,
          bool PERSIST = false>
__global__ __launch_bounds__(WM * WN * 64, 1) __attribute__((amdgpu_waves_per_eu(WM * WN / 4, WM * WN / 4))) void gemm_i8_kernel(
    const int8_t* __restrict__ Ares, const int8_t* __restrict__ Bres, int m_pad, int n_pad, int q_pad, GemmConsts c,
    int32_t* __restrict__ Ct, uint8_t* __restrict__ rt, const int4* __restrict__ plan, int k_begin, int k_slices,
    int nblocks) {
  constexpr int NW = WM * WN;
  constexpr int CPR = BK / 16;                  // 16-byte chunks per tile row
  constexpr int ROWS_PER_KB = 1024 / BK;        // tile rows filled by one wavefront load
  constexpr int A_LOADS = BM * BK / 1024 / NW;  // wavefront loads per slice
  constexpr int B_LOADS = BN * BK / 1024 / NW;
  constexpr int LPW = A_LOADS + B_LOADS;        // loads per wavefront per slice
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int MT = 16;                        // MFMA tile (see above)
  constexpr int KSTEP = 1024 / MT;              // K bytes per MFMA: 64
  constexpr int CPS = KSTEP / 16;               // 16-byte K chunks per step
  constexpr int ACC_N = MT * MT / 64;           // accumulators per lane per tile: 4
  constexpr int FM = WTM / MT, FN = WTN / MT;
  constexpr int NKS = BK / KSTEP;               // K steps per slice
  constexpr int NF = FM + FN;                   // fragments per step
  constexpr int SLOTS = FM * FN;                // MFMAs per step
  constexpr int RS = SLOTS / NF;                // slots per fragment read (four wavefronts)
  constexpr bool EIGHT = NW == 8;
  static_assert(NW == 4 || (EIGHT && FM == 8 && FN == 4), "four wavefronts, or eight of 128 x 64");
  static_assert(EIGHT || (WRITE_RT && !WRITE_CT), "int32 output runs eight wavefronts");
  static_assert(A_LOADS >= 1 && B_LOADS >= 1 && BM * BK % (1024 * NW) == 0, "tile/wave mismatch");
  static_assert((EIGHT || SLOTS % NF == 0) && NKS >= 2, "slot plan: whole reads per step, two steps per slice");
  static_assert(load_slot(EIGHT, RS, LPW - 1) < SLOTS * NKS, "every load has a slot in its window");
  // loads of a slice issued in the window before it: those whose slot falls
  // in the last step of the slice before (all of them)
  constexpr int HALF_LOADS = early_loads(EIGHT, RS, LPW, SLOTS);
  static_assert(HALF_LOADS == LPW, "prologue load count");
  typedef int acc_t __attribute__((ext_vector_type(ACC_N)));

  // Staged residue output: the words are first placed in LDS as the tile's
  // columns (BM bytes each, stride CS), then each wavefront writes whole
  // column segments with 16-byte stores, four columns per instruction.  A
  // direct store from the MFMA layout writes 32 scattered 8-byte pieces per
  // instruction.  The staging area is the operand buffers (free after the K
  // loop), or, in the persistent form, buffer 1 and what follows it, so that
  // the next tile's first slice can land in buffer 0 meanwhile.
  constexpr bool STAGED = WRITE_RT && !WRITE_CT && !ACC_RT;
  // Residue-only output starts the accumulators at -(m_t - 1)/2 (0 for
  // m_t = 256), which lets the epilogue reduce each entry with one rounding
  // fma and one 24-bit multiply-add (mod_product_biased).
  constexpr bool BIASED = WRITE_RT && !WRITE_CT;
  static_assert(!PERSIST || (STAGED && !MULTI), "persistent form: residue-only products");
  constexpr int CS = BM + 16;  // 16-byte aligned; consecutive columns start 4 banks apart
  constexpr int OPERANDS = 2 * (BM + BN) * BK;
  constexpr int STAGE_OFF = PERSIST ? (BM + BN) * BK : 0;
  constexpr int SMEM = STAGED && STAGE_OFF + BN * CS > OPERANDS ? STAGE_OFF + BN * CS : OPERANDS;
  static_assert(!STAGED || (BM % 256 == 0 && BN % (4 * NW) == 0), "whole column segments per store");

  __shared__ __attribute__((aligned(1024))) int8_t smem[SMEM];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WN, wn = wave % WN;

  const int tiles_m = m_pad / BM, tiles_n = n_pad / BN;
  const int nplanes = nblocks / (tiles_m * tiles_n);
  const long a_plane = (long)m_pad * q_pad, b_plane = (long)n_pad * q_pad;
  const int nk = q_pad / BK;  // K slices per product

  // The tile of linear block id L (one per block, or L = blockIdx.x +
  // r gridDim.x, r = 0, 1, ... in the persistent form -- the same XCD as in
  // a grid of nblocks blocks): its modulus or plan entry t, output corner,
  // output plane, operand panels and K slices.  Operand planes: (t, t) once,
  // or (a0 + u, b0 - u) for u < count.
  int t, m0, n0, out_t, kfirst, nkt;
  const int8_t* Ag;
  const int8_t* Bg;
  auto set_tile = [&](int L) {
    int tt, mi, nj;
    tile_of_block<4>(L, nplanes, tiles_m, tiles_n, tt, mi, nj);
    m0 = mi * BM;
    n0 = nj * BN;
    out_t = tt;  // output plane
    int part = 0;
    if (!MULTI) {
      part = tt / c.s;  // K part of modulus tt
      tt -= part * c.s;
    }
    int a0 = tt, b0 = tt, count = 1;
    if (MULTI) {
      const int4 pl = plan[tt];
      a0 = pl.x;
      b0 = pl.y;
      count = pl.z;
      out_t = pl.w;
    }
    t = tt;
    Ag = Ares + (long)a0 * a_plane + (long)m0 * q_pad;
    Bg = Bres + (long)b0 * b_plane + (long)n0 * q_pad;
    kfirst = k_begin + part * k_slices;                          // first K slice of this block
    nkt = MULTI ? nk * count : min(k_slices, nk - kfirst);       // K slices walked
  };
  int L = blockIdx.x;
  set_tile(L);

  // A wavefront load fills 1 KB of LDS = ROWS_PER_KB whole tile rows, lane l
  // landing in row l / CPR, physical chunk l mod CPR.  The swizzle depends on
  // row mod 16, so the source offset differs between even and odd 1 KB blocks.
  const int lrow_in_kb = lane / CPR;
  const int lane_src0 = lrow_in_kb * q_pad + (((lane % CPR) ^ swz<BK>(lrow_in_kb)) * 16);
  const int lane_src1 = lrow_in_kb * q_pad + (((lane % CPR) ^ swz<BK>(lrow_in_kb + ROWS_PER_KB)) * 16);
  const long kb_stride = (long)ROWS_PER_KB * q_pad;  // source distance of consecutive 1 KB loads

  // load li (A blocks first, then B) of walked slice kk into buffer kk mod 2
  auto load1 = [&](int kk, int li) {
    int8_t* As = smem + (kk & 1) * (BM + BN) * BK;
    int8_t* Bs = As + BM * BK;
    const int8_t* ga = Ag;
    const int8_t* gb = Bg;
    int k0 = (kfirst + kk) * BK;
    if (MULTI) {
      const int u = kk / nk;
      k0 = (kk - u * nk) * BK;
      ga += u * a_plane;
      gb -= u * b_plane;
    }
    if (li < A_LOADS) {
      const int blk = wave * A_LOADS + li;
      __builtin_amdgcn_global_load_lds(ga + blk * kb_stride + k0 + ((blk & 1) ? lane_src1 : lane_src0),
                                       As + blk * 1024, 16, 0, 0);
    } else {
      const int blk = wave * B_LOADS + (li - A_LOADS);
      __builtin_amdgcn_global_load_lds(gb + blk * kb_stride + k0 + ((blk & 1) ? lane_src1 : lane_src0),
                                       Bs + blk * 1024, 16, 0, 0);
    }
  };

  const int lrow = lane % MT;
  const int lkc = lane / MT;  // K chunk within a step
  // fragment f of step ks in buffer buf: f < FN are B columns, the rest A rows
  auto read1 = [&](int buf, int ks, int f) -> v4i {
    const int8_t* As = smem + buf * (BM + BN) * BK;
    const int8_t* Bs = As + BM * BK;
    const int kc = ks * CPS + lkc;
    if (f < FN) {
      const int row = wn * WTN + f * MT + lrow;
      return *reinterpret_cast<const v4i*>(&Bs[row * BK + ((kc ^ swz<BK>(row)) * 16)]);
    }
    const int row = wm * WTM + (f - FN) * MT + lrow;
    return *reinterpret_cast<const v4i*>(&As[row * BK + ((kc ^ swz<BK>(row)) * 16)]);
  };

  // this plane's modulus, selected without indexing the by-value argument
  // dynamically (which would copy it to scratch)
  auto modulus = [&]() {
    int mt = c.m[0];
#pragma unroll
    for (int u = 1; u < OZGEMM_S_MAX; ++u) mt = (u == t) ? c.m[u] : mt;
    return mt;
  };
  auto reset_acc = [&](acc_t (&a)[FM][FN]) {
    acc_t start = {};
    if (BIASED) start += mod_bias(modulus()).bias;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) a[i][j] = start;
  };

  acc_t acc[FM][FN];
  reset_acc(acc);

  // The window after barrier kt - 1 holds SLOTS NKS slots: the last step of
  // slice kt - 1 (slots 0..SLOTS-1), then steps 0..NKS-2 of slice kt.  Its
  // loads fetch slice kt + 1 into the buffer retired by that barrier; load li
  // goes after slot RS li + 1.  The prologue stands in for the part of
  // window 0 that precedes slice 0.
#pragma unroll
  for (int li = 0; li < LPW; ++li) load1(0, li);
  if (nkt > 1) {
#pragma unroll
    for (int li = 0; li < LPW; ++li)
      if (load_slot(EIGHT, RS, li) < SLOTS) load1(1, li);
    wait_vmcnt<HALF_LOADS>();  // slice 0 (loads return in order)
  } else {
    wait_vmcnt<0>();
  }
  __builtin_amdgcn_s_barrier();

  const long plane = (long)m_pad * n_pad;
  uint8_t* stage = reinterpret_cast<uint8_t*>(smem + STAGE_OFF);
  while (true) {
    v4i cur[NF], nxt[NF];
#pragma unroll
    for (int f = 0; f < NF; ++f) cur[f] = read1(0, 0, f);
    // The slice loop is entered, and each iteration ends, with no LDS read in
    // flight.  The compiler places a full lgkmcnt wait at the loop head;
    // with each slot's MFMA issued before its read, that wait then costs
    // nothing, where it used to follow the step's first read and take a whole
    // LDS latency once per slice (1-1.5% of the product at 8192^3).
    __builtin_amdgcn_s_waitcnt(0xc07f);

    for (int kt = 0; kt < nkt; ++kt) {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const bool last = ks == NKS - 1;
        const int lslice = last ? kt + 2 : kt + 1;  // slice fetched in this step's window
        if (last) {
          __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's reads of slice kt are done
          wait_vmcnt<0>();                     // this wave's loads of slice kt + 1 have landed
          __builtin_amdgcn_s_barrier();
        }
        const int rbuf = last ? (kt + 1) & 1 : kt & 1;  // (past the end: read, unused)
        const int rks = last ? 0 : ks + 1;
#pragma unroll
        for (int r = 0; r < SLOTS; ++r) {
          const int i = r / FN, j = r % FN;
          acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(cur[FN + i], cur[j], acc[i][j], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);  // the slot's MFMA issues before its read
#pragma unroll
          for (int f = 0; f < NF; ++f)
            if (read_slot(EIGHT, RS, FN, f) == r) nxt[f] = read1(rbuf, rks, f);
          const int slot = last ? r : SLOTS + ks * SLOTS + r;
#pragma unroll
          for (int li = 0; li < LPW; ++li)
            if (load_slot(EIGHT, RS, li) == slot && lslice < nkt) load1(lslice, li);
          __builtin_amdgcn_sched_barrier(0);
        }
        if (last) __builtin_amdgcn_s_waitcnt(0xc07f);  // no LDS read in flight (see above)
#pragma unroll
        for (int f = 0; f < NF; ++f) cur[f] = nxt[f];
      }
    }
    wait_vmcnt<0>();  // no load into LDS may outlive the block

    // ---- epilogue: int32 planes and/or residues mod m_t ----
    const int mt = modulus();
    const double md = (double)mt, inv = 1.0 / md;  // correctly rounded
    const ModBias mb = mod_bias(mt);
    const int em0 = m0, en0 = n0, eout = out_t;    // the finished tile
    bool more = false;
    if (STAGED) {
      __builtin_amdgcn_s_waitcnt(0xc07f);  // this wave's last LDS reads are done
      __builtin_amdgcn_s_barrier();        // and every other wave's
      if (PERSIST) {
        // the next tile's first slice lands in buffer 0 while this one's
        // residues are reduced and written
        more = L + (int)gridDim.x < nblocks;
        if (more) {
          L += gridDim.x;
          set_tile(L);
#pragma unroll
          for (int li = 0; li < LPW; ++li) load1(0, li);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int lcol = wn * WTN + j * MT + lane % MT;
        const int col = en0 + lcol;
#pragma unroll
        for (int g = 0; g < ACC_N / 4; ++g) {  // four consecutive rows each
          const int lrow4 = wm * WTM + i * MT + 8 * g + 4 * (lane / MT);
          const int row = em0 + lrow4;
          const long off = (long)eout * plane + (long)col * m_pad + row;
          const acc_t& v = acc[i][j];
          if (WRITE_CT) *reinterpret_cast<v4i*>(Ct + off) = v4i{v[4 * g], v[4 * g + 1], v[4 * g + 2], v[4 * g + 3]};
          if (WRITE_RT) {
            uint32_t r0, r1, r2, r3;
            if (BIASED) {  // residues in the low bytes
              r0 = mod_product_biased(from_agpr(v[4 * g]), mb.negm, inv, mb.magic);
              r1 = mod_product_biased(from_agpr(v[4 * g + 1]), mb.negm, inv, mb.magic);
              r2 = mod_product_biased(from_agpr(v[4 * g + 2]), mb.negm, inv, mb.magic);
              r3 = mod_product_biased(from_agpr(v[4 * g + 3]), mb.negm, inv, mb.magic);
            } else {
              r0 = mod_product(v[4 * g], md, inv);
              r1 = mod_product(v[4 * g + 1], md, inv);
              r2 = mod_product(v[4 * g + 2], md, inv);
              r3 = mod_product(v[4 * g + 3], md, inv);
            }
            if (ACC_RT) {  // add the residues of the earlier K blocks, mod m_t
              r0 &= 0xffu;
              r1 &= 0xffu;
              r2 &= 0xffu;
              r3 &= 0xffu;
              const uint32_t old = *reinterpret_cast<const uint32_t*>(rt + off);
              r0 += old & 0xffu;
              r1 += (old >> 8) & 0xffu;
              r2 += (old >> 16) & 0xffu;
              r3 += old >> 24;
              r0 = r0 >= (uint32_t)mt ? r0 - mt : r0;
              r1 = r1 >= (uint32_t)mt ? r1 - mt : r1;
              r2 = r2 >= (uint32_t)mt ? r2 - mt : r2;
              r3 = r3 >= (uint32_t)mt ? r3 - mt : r3;
            }
            const uint32_t word = low_bytes(r0, r1, r2, r3);
            if (STAGED)
              *reinterpret_cast<uint32_t*>(stage + lcol * CS + lrow4) = word;
            else
              *reinterpret_cast<uint32_t*>(rt + off) = word;
          }
        }
        // keep the scheduler from hoisting every accumulator out of AGPRs at
        // once: a barrier after every 16 accumulators
        if ((j + 1) * ACC_N % 16 == 0) __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (STAGED) {
      __builtin_amdgcn_s_waitcnt(0xc07f);
      __builtin_amdgcn_s_barrier();
      // wavefront w writes tile columns [w BN/NW, (w+1) BN/NW): 16 lanes per
      // column, 16 bytes each
      constexpr int COLS_PER_WAVE = BN / NW, LANES_PER_COL = BM / 16;
      static_assert(!STAGED || 64 % LANES_PER_COL == 0, "whole columns per store");
      constexpr int COLS_PER_STORE = 64 / LANES_PER_COL;
#pragma unroll
      for (int it = 0; it < COLS_PER_WAVE / COLS_PER_STORE; ++it) {
        const int lcol = wave * COLS_PER_WAVE + it * COLS_PER_STORE + lane / LANES_PER_COL;
        const int rch = (lane % LANES_PER_COL) * 16;
        const uint4 v = *reinterpret_cast<const uint4*>(stage + lcol * CS + rch);
        *reinterpret_cast<uint4*>(rt + (long)eout * plane + (long)(en0 + lcol) * m_pad + em0 + rch) = v;
      }
    }
    if (!PERSIST || !more) break;

    // next tile: every wave has read its staged columns out of buffer 1
    // before the first half of slice 1 is loaded there
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_s_barrier();
    if (nkt > 1)
#pragma unroll
      for (int li = 0; li < LPW; ++li)
        if (load_slot(EIGHT, RS, li) < SLOTS) load1(1, li);
    reset_acc(acc);
    // Wait for slice 0 only: it went out before this tile's stores and
    // slice 1's loads, and loads and stores retire from the counter in issue
    // order.  The stores and slice 1 complete under step 0 of the next tile
    // and are waited for at its first barrier.  (16384^2 x 1024: 1.6% off the
    // product, against waiting for everything here.)
    constexpr int STORES = STAGED ? (BN / NW) / (64 / (BM / 16)) : 0;  // 16-byte stores per wave above
    if (nkt > 1)
      wait_vmcnt<STORES + HALF_LOADS>();
    else
      wait_vmcnt<STORES>();
    __builtin_amdgcn_s_barrier();
  }
}

// Sum of the K parts' residues (gemm_grid.h): dst plane t = (sum over p < P
// of src plane p s + t) mod m_t, 16 bytes per thread.  The bytes of a word are
// summed in two 16-bit lanes each (even and odd bytes; P <= 64 keeps a sum
// below 2^16).  dst may be src: plane t of part 0 is read by the same thread
// before it is written, and no other thread touches it.
__global__ __launch_bounds__(256) void rt_parts_reduce_kernel(const uint8_t* __restrict__ src, uint8_t* dst,
                                                             long plane, int P, GemmConsts c) {
  const long chunks = plane / 16;
  const long gid = (long)blockIdx.x * 256 + threadIdx.x;
  if (gid >= chunks * c.s) return;
  const int t = (int)(gid / chunks);
  const long off = (gid - (long)t * chunks) * 16;
  int mt = c.m[0];
#pragma unroll
  for (int u = 1; u < OZGEMM_S_MAX; ++u) mt = (u == t) ? c.m[u] : mt;
  const double md = (double)mt, inv = 1.0 / md;
  uint32_t ev[4] = {0, 0, 0, 0}, od[4] = {0, 0, 0, 0};
  for (int p0 = 0; p0 < P; p0 += 8) {
    uint4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {  // all loads first; a clamped index past P is loaded but not added
      const int p = min(p0 + i, P - 1);
      v[i] = *reinterpret_cast<const uint4*>(src + ((long)p * c.s + t) * plane + off);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (p0 + i < P) {
        const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          ev[k] += w[k] & 0x00ff00ffu;
          od[k] += (w[k] >> 8) & 0x00ff00ffu;
        }
      }
    }
  }
  uint32_t out[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t r0 = mod_product((int32_t)(ev[k] & 0xffffu), md, inv);
    const uint32_t r2 = mod_product((int32_t)(ev[k] >> 16), md, inv);
    const uint32_t r1 = mod_product((int32_t)(od[k] & 0xffffu), md, inv);
    const uint32_t r3 = mod_product((int32_t)(od[k] >> 16), md, inv);
    out[k] = r0 | (r1 << 8) | (r2 << 16) | (r3 << 24);
  }
  *reinterpret_cast<uint4*>(dst + (long)t * plane + off) = uint4{out[0], out[1], out[2], out[3]};
}

}  // namespace

hipError_t launch_gemm(const int8_t* Ares, const int8_t* Bres, int m_pad, int n_pad, int q_pad, const GemmConsts& c,
                       int32_t* Ct, uint8_t* rt, const SplitChoice& split, uint8_t* parts, int cus,
                       hipStream_t st) {
  constexpr int BM = 256, BN = 256, BK = 128, WM = 2, WN = 2, WN8 = 4;  // four or eight wavefronts
  static_assert(BK == SPLIT_K_SLICE, "K parts are counted in kernel slices");
  if (m_pad % BM || n_pad % BN || q_pad % BK) return hipErrorInvalidValue;
  const int tiles = (n_pad / BN) * (m_pad / BM);
  const int nblocks = tiles * c.s;
  const dim3 grid(nblocks), block(WM * WN * 64);
  const int nk = q_pad / BK;
  // residue-only products walk their tiles with one block per compute unit
  // (the persistent form) when there are more tiles than units; blocks that
  // walk few K slices run eight wavefronts
  auto launch_rt = [&](uint8_t* out, int total, int per) {
    const bool eight = per <= EIGHT_WAVE_MAX_SLICES;
    if (cus > 0 && total > cus && eight)
      hipLaunchKernelGGL((gemm_i8_kernel<BM, BN, BK, WM, WN8, false, true, false, false, true>), dim3(cus),
                         dim3(WM * WN8 * 64), 0, st, Ares, Bres, m_pad, n_pad, q_pad, c, Ct, out, nullptr, 0, per,
                         total);
    else if (cus > 0 && total > cus)
      hipLaunchKernelGGL((gemm_i8_kernel<BM, BN, BK, WM, WN, false, true, false, false, true>), dim3(cus), block,
                         0, st, Ares, Bres, m_pad, n_pad, q_pad, c, Ct, out, nullptr, 0, per, total);
    else if (eight)
      hipLaunchKernelGGL((gemm_i8_kernel<BM, BN, BK, WM, WN8, false, true, false>), dim3(total),
                         dim3(WM * WN8 * 64), 0, st, Ares, Bres, m_pad, n_pad, q_pad, c, Ct, out, nullptr, 0, per,
                         total);
    else
      hipLaunchKernelGGL((gemm_i8_kernel<BM, BN, BK, WM, WN, false, true, false>), dim3(total), block, 0, st,
                         Ares, Bres, m_pad, n_pad, q_pad, c, Ct, out, nullptr, 0, per, total);
  };
  if (Ct == nullptr && rt != nullptr && split.parts > 1) {
    // K parts into the part planes, then their sum mod m_t into rt
    const int P = split.parts, per = split.slices;
    if (parts == nullptr || P > SPLIT_MAX || per < 1 || (long)(P - 1) * per >= nk || (long)P * per < nk ||
        (q_pad >= OZGEMM_Q_LIMIT && per > KBLOCK_K / BK))
      return hipErrorInvalidValue;
    launch_rt(parts, nblocks * P, per);
    const long plane = (long)m_pad * n_pad;
    const long threads = plane / 16 * c.s;
    hipLaunchKernelGGL(rt_parts_reduce_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, parts, rt,
                       plane, P, c);
    return hipGetLastError();
  }
  if (q_pad >= OZGEMM_Q_LIMIT && Ct == nullptr && rt != nullptr) {
    // block products; int32 C_t planes are only asked for while q < 2^17,
    // where one launch is exact (the padding is zero)
    constexpr int per = KBLOCK_K / BK;
    for (int k0 = 0; k0 < nk; k0 += per) {
      const int cnt = std::min(per, nk - k0);
      if (k0 == 0)
        hipLaunchKernelGGL((gemm_i8_kernel<BM, BN, BK, WM, WN, false, true, false, false>), grid, block, 0, st,
                           Ares, Bres, m_pad, n_pad, q_pad, c, Ct, rt, nullptr, k0, cnt, nblocks);
      else
        hipLaunchKernelGGL((gemm_i8_kernel<BM, BN, BK, WM, WN, false, true, false, true>), grid, block, 0, st,
                           Ares, Bres, m_pad, n_pad, q_pad, c, Ct, rt, nullptr, k0, cnt, nblocks);
    }
    return hipGetLastError();
  }
  // int32 planes (the stage entry point's debug output): eight wavefronts
  if (Ct != nullptr && rt != nullptr)
    hipLaunchKernelGGL((gemm_i8_kernel<BM, BN, BK, WM, WN8, true, true, false>), grid, dim3(WM * WN8 * 64), 0, st,
                       Ares, Bres, m_pad, n_pad, q_pad, c, Ct, rt, nullptr, 0, nk, nblocks);
  else if (Ct != nullptr)
    hipLaunchKernelGGL((gemm_i8_kernel<BM, BN, BK, WM, WN8, true, false, false>), grid, dim3(WM * WN8 * 64), 0, st,
                       Ares, Bres, m_pad, n_pad, q_pad, c, Ct, rt, nullptr, 0, nk, nblocks);
  else if (rt != nullptr)
    launch_rt(rt, nblocks, nk);
  return hipGetLastError();
}

hipError_t launch_gemm_multi(const int8_t* Aplanes, const int8_t* Bplanes, int m_pad, int n_pad, int q_pad,
                             const int4* plan, int nout, int32_t* P, hipStream_t st) {
  constexpr int BM = 256, BN = 256, BK = 128, WM = 2, WN = 4;  // eight wavefronts
  if (m_pad % BM || n_pad % BN || q_pad % BK || nout < 1) return hipErrorInvalidValue;
  GemmConsts none{};
  none.s = 1;
  none.m[0] = 2;
  const int nblocks = (n_pad / BN) * (m_pad / BM) * nout;
  hipLaunchKernelGGL((gemm_i8_kernel<BM, BN, BK, WM, WN, true, false, true>), dim3(nblocks),
                     dim3(WM * WN * 64), 0, st, Aplanes, Bplanes, m_pad, n_pad, q_pad, none, P, nullptr, plan, 0, 0,
                     nblocks);
  return hipGetLastError();
}

}  // namespace oz
