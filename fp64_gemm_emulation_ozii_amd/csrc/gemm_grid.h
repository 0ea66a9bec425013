// Block grid of the int8 product launches (host and device code; a CPU test
// driver builds it too): which plane and output tile a block computes, and
// into how many K parts a Scheme II product is cut.
//
// K parts.  A product launch runs one block per (modulus, 256 x 256 output
// tile).  When moduli x tiles is small against the compute units -- a skinny
// output with a long inner dimension -- the K range is cut into P parts and
// every (part, modulus, tile) gets a block.  Part p writes the residue of its
// partial product mod m_t into plane p s + t, and a reduction adds the P
// residues of each entry mod m_t.  The sum of the parts is the whole product,
// so the result is C_t mod m_t as before.  A part is an exact int32 product
// while it spans at most 2^16 K entries (|.| <= 2^16 2^14 < 2^31; Ozaki II
// notes §6, block products), so for q >= 2^17 the parts also replace the
// sequential launches over K blocks whenever their planes fit.
#pragma once

#include <algorithm>

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

// Map the linear block id b to (plane t, tile row mi, tile column nj) of a
// launch over nplanes planes of tiles_m x tiles_n tiles.
//
// Blocks go to the 8 XCDs round-robin (block b runs on XCD b mod 8) and each
// XCD has its own L2.  The planes are walked one at a time, so all XCDs work
// on the same plane and its operands stay in the shared last-level cache;
// inside a plane each XCD takes a contiguous eighth of the tiles, walked in
// groups of GROUP_M tile rows, so the blocks running on one XCD at a time
// share A row panels and B column panels in its L2.  A plane of at most 32
// tiles (an XCD runs 32 blocks at once) goes whole to one XCD instead, when
// the planes divide evenly among the XCDs, so that every A and B panel of the
// plane is fetched once into that XCD's L2.
template <int GROUP_M>
__host__ __device__ __forceinline__ void tile_of_block(int b, int nplanes, int tiles_m, int tiles_n, int& t,
                                                       int& mi, int& nj) {
  const int per_plane = tiles_m * tiles_n;
  int tile;
  if (per_plane <= 32 && nplanes % 8 == 0) {
    const int j = b / 8;  // the j-th block of XCD b mod 8
    t = (j / per_plane) * 8 + b % 8;
    tile = j % per_plane;
  } else {
    t = b / per_plane;
    const int w = b % per_plane;
    tile = (per_plane % 8 == 0) ? (w % 8) * (per_plane / 8) + w / 8 : w;
  }
  const int group = tile / (GROUP_M * tiles_n);
  const int first_m = group * GROUP_M;
  const int rest = tiles_m - first_m;
  const int gm = rest < GROUP_M ? rest : GROUP_M;
  const int in_group = tile % (GROUP_M * tiles_n);
  mi = first_m + in_group % gm;
  nj = in_group / gm;
}

constexpr int SPLIT_K_SLICE = 128;       // K entries per slice of the product kernel
constexpr int SPLIT_MAX = 64;            // the reduction sums up to 64 residues in 16-bit lanes
constexpr int SPLIT_MIN_SLICES = 16;     // nk >= P x 16: parts average >= 2048 K entries, unless exactness needs more
constexpr long SPLIT_BLOCKS = 2048;      // parts x moduli x tiles: bounds the part planes to 2048 x 64 KB
constexpr int SPLIT_EXACT_SLICES = 512;  // 2^16 K entries: the longest exact part

struct SplitChoice {
  int parts;   // 1: one block per (modulus, tile); 0: sequential K-block launches
  int slices;  // K slices per part (the last part may hold fewer)
};

inline long split_ceil_div(long a, long b) { return (a + b - 1) / b; }

// Modelled time of a launch of P parts of `per` slices, in units of one
// block's K slice.  Blocks run in waves of `cus`; each block pays a fixed
// prologue/epilogue of about 6 slices.  Blocks that run together share their
// operand panels in L2 when a plane spans >= 64 tiles (an XCD takes eighths of
// a plane) or when whole planes of <= 32 tiles sit on one XCD (P s a multiple
// of 8); otherwise the operand traffic costs about a quarter more.  The part
// planes cost one write, one read and the reduction, about 0.02 slice per
// block over the whole chip.
inline double split_cost(int P, int per, int tiles, int s, int cus) {
  const long blocks = (long)P * s * tiles;
  const long waves = split_ceil_div(blocks, cus);
  const bool shared = tiles >= 64 || (tiles <= 32 && (P * s) % 8 == 0);
  return (double)waves * (per + 6.0) * (shared ? 1.0 : 1.25) + (P > 1 ? 0.02 * (double)blocks : 0.0);
}

// Parts for a residue-only product of `tiles` output tiles per modulus, s
// moduli and nk K slices, on `cus` compute units, with room for cap_planes
// output planes.  One launch is exact while nk < 1024 (q_pad < 2^17); beyond
// that at least ceil(nk / 512) parts are needed, or the sequential K blocks.
// Splitting is taken only when the model gains 5% over one part.
inline SplitChoice choose_splits(int tiles, int s, int nk, int cus, long cap_planes) {
  const int pmin = nk >= 2 * SPLIT_EXACT_SLICES ? (int)split_ceil_div(nk, SPLIT_EXACT_SLICES) : 1;
  SplitChoice best{pmin == 1 ? 1 : 0, pmin == 1 ? nk : 0};
  double best_cost = pmin == 1 ? 0.95 * split_cost(1, nk, tiles, s, cus) : 0.0;
  if (tiles < 1 || s < 1 || nk < 1 || cus < 1) return best;
  for (int P = std::max(2, pmin); P <= SPLIT_MAX; ++P) {
    if (nk < P * SPLIT_MIN_SLICES && P > pmin) break;
    const int per = (int)split_ceil_div(nk, P);
    if ((long)P * s * tiles > SPLIT_BLOCKS || (long)P * s > cap_planes) break;
    if (split_ceil_div(nk, per) != P) continue;  // the last part would be empty
    const double c = split_cost(P, per, tiles, s, cus);
    if (best.parts == 0 || c < best_cost) {
      best = SplitChoice{P, per};
      best_cost = c;
    }
  }
  return best;
}

// Bytes of part planes a configuration must hold so that every choice above
// fits: none while no product can have 2 x SPLIT_MIN_SLICES slices.
inline long split_region_bytes(int max_nk, int tile_bytes) {
  return max_nk >= 2 * SPLIT_MIN_SLICES ? SPLIT_BLOCKS * (long)tile_bytes : 0;
}

}  // namespace oz
