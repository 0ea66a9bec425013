// Host driver for the product-residue header: reads "m count" then count
// int32 values on stdin and prints v mod m as computed by mod_product.
#include <cstdio>
#include <cstdint>

#include "../fp64_gemm_emulation_ozii_amd/csrc/prod_mod.h"

int main() {
  int m, count;
  while (std::scanf("%d %d", &m, &count) == 2) {
    const double md = (double)m, inv = 1.0 / md;
    for (int i = 0; i < count; ++i) {
      long long v;
      if (std::scanf("%lld", &v) != 1) return 1;
      std::printf("%u\n", oz::mod_product((int32_t)v, md, inv));
    }
  }
  return 0;
}
