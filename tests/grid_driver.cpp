// Host driver for the product launch grid header.  Reads commands on stdin:
//   map <nplanes> <tiles_m> <tiles_n>   -> one line "t mi nj" per block id
//   split <tiles> <s> <nk> <cus> <cap>  -> "parts slices region_bytes"
#include <cstdio>
#include <cstring>

#include "../fp64_gemm_emulation_ozii_amd/csrc/gemm_grid.h"

int main() {
  char cmd[16];
  while (std::scanf("%15s", cmd) == 1) {
    if (std::strcmp(cmd, "map") == 0) {
      int np, tm, tn;
      if (std::scanf("%d %d %d", &np, &tm, &tn) != 3) return 1;
      for (int b = 0; b < np * tm * tn; ++b) {
        int t, mi, nj;
        oz::tile_of_block<4>(b, np, tm, tn, t, mi, nj);
        std::printf("%d %d %d\n", t, mi, nj);
      }
    } else if (std::strcmp(cmd, "split") == 0) {
      int tiles, s, nk, cus;
      long cap;
      if (std::scanf("%d %d %d %d %ld", &tiles, &s, &nk, &cus, &cap) != 5) return 1;
      const oz::SplitChoice c = oz::choose_splits(tiles, s, nk, cus, cap);
      std::printf("%d %d %ld\n", c.parts, c.slices, oz::split_region_bytes(nk, 256 * 256));
    } else {
      return 1;
    }
  }
  return 0;
}
