// Host driver for the product-residue header: reads "m count" then count
// int32 values v on stdin and prints, per value, v mod m as computed by
// mod_product, and the low byte of mod_product_biased on the accumulator
// v - h that the biased form starts from (or -1 where v - h leaves int32).
#include <cstdio>
#include <cstdint>

#include "../fp64_gemm_emulation_ozii_amd/csrc/prod_mod.h"

int main() {
  int m, count;
  while (std::scanf("%d %d", &m, &count) == 2) {
    const double md = (double)m, inv = 1.0 / md;
    const oz::ModBias mb = oz::mod_bias(m);
    for (int i = 0; i < count; ++i) {
      long long v;
      if (std::scanf("%lld", &v) != 1) return 1;
      const long long acc = v + mb.bias;
      long long biased = -1;
      if (acc >= INT32_MIN && acc <= INT32_MAX)
        biased = oz::mod_product_biased((int32_t)acc, mb.negm, inv, mb.magic) & 0xffu;
      std::printf("%u %lld\n", oz::mod_product((int32_t)v, md, inv), biased);
    }
  }
  return 0;
}
