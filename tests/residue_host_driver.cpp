// Host driver for csrc/residue_arith.h, the per-entry arithmetic the residue
// kernels inline.  Each input line is "<form> <m> <A' as IEEE bits in hex>
// <plant>"; the output line is the symmetric residue the header computes.
//   form 0: |A'| < 2^50 (residue_narrow)
//   form 1: |A'| < 2^53 (split_wide<false>, residue_wide<false>)
//   form 2: |A'| < 2^78 (split_wide<true>, residue_wide<true>)
//   plant 1: 2^51 mod m in place of 2^52 mod m; plant 2: form 0's reduction
//   applied to A' as it is (no split).  Both are planted mistakes the test
//   must see.
// The per-modulus constants are made as the library's host code makes them:
// RN(1/m), 2^26 mod m and 2^52 mod m.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "../fp64_gemm_emulation_ozii_amd/csrc/residue_arith.h"

int main() {
  int form, m, plant;
  char hex[32];
  while (std::scanf("%d %d %31s %d", &form, &m, hex, &plant) == 4) {
    const uint64_t bits = std::strtoull(hex, nullptr, 16);
    double a;
    std::memcpy(&a, &bits, sizeof a);
    const double md = (double)m, inv = 1.0 / md;
    const double c26 = (double)((1ull << 26) % (uint64_t)m);
    const double c52 = (double)((1ull << (plant == 1 ? 51 : 52)) % (uint64_t)m);
    int r;
    if (form == 0 || plant == 2) {
      r = (int32_t)oz::residue_narrow(a, a + 0x1.8p52, md, inv);
    } else if (form == 1) {
      double a1 = 0.0, a2 = 0.0;
      oz::split_wide<false>(a, a1, a2);
      r = oz::residue_wide<false>(a, a1, a2, c26, c52, md, inv);
    } else {
      double a1 = 0.0, a2 = 0.0;
      oz::split_wide<true>(a, a1, a2);
      r = oz::residue_wide<true>(a, a1, a2, c26, c52, md, inv);
    }
    std::printf("%d\n", r);
  }
  return 0;
}
