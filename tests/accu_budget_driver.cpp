// Host driver for the OS II-accu budget comparison (csrc/accu_budget.h): reads
// "vtop bv count" then count values of N, prints floor(log2(V / N)) for each.
#include <cstdio>
#include <cstdint>

#include "../fp64_gemm_emulation_ozii_amd/csrc/accu_budget.h"

int main() {
  unsigned long long vtop = 0, N = 0;
  int bv = 0, count = 0;
  while (std::scanf("%llu %d %d", &vtop, &bv, &count) == 3) {
    for (int c = 0; c < count; ++c) {
      if (std::scanf("%llu", &N) != 1) return 1;
      std::printf("%d\n", oz::floor_log2_ratio((uint64_t)N, (uint64_t)vtop, bv));
    }
  }
  return 0;
}
