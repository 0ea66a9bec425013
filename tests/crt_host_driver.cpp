// Host driver for the CRT reconstruction header: reads cases on stdin and
// prints the resulting doubles as 16-digit hex bit patterns.
//   line 1: W L  M-limbs(5)  half-limbs(5)  halfM(hex bits)  invM(hex bits)
//           (W = limb width, 32 or 40 bits)
//   line 2: count
//   then per case: scale S_0 .. S_{L-1}   (S as decimal integers < 2^53)
#include <cstdio>
#include <cstdint>
#include <cstring>

#include "../fp64_gemm_emulation_ozii_amd/csrc/crt_reconstruct.h"

static double from_bits(unsigned long long b) {
  double d;
  std::memcpy(&d, &b, 8);
  return d;
}

template <int L, int W>
static void run(const oz::CrtModulus& K, int count) {
  for (int i = 0; i < count; ++i) {
    int scale;
    if (std::scanf("%d", &scale) != 1) return;
    double S[L];
    for (int l = 0; l < L; ++l) {
      long long v;
      if (std::scanf("%lld", &v) != 1) return;
      S[l] = (double)v;
    }
    const double r = W == 40 ? oz::reconstruct40<(L <= 3 ? L : 3)>(S, K, scale) : oz::reconstruct_limbs<L>(S, K, scale);
    unsigned long long b;
    std::memcpy(&b, &r, 8);
    std::printf("%016llx\n", b);
  }
}

int main() {
  int W, L;
  oz::CrtModulus K;
  unsigned long long hb, ib;
  if (std::scanf("%d %d", &W, &L) != 2) return 1;
  if ((W != 32 && W != 40) || (W == 40 && L > 3)) return 1;
  for (int l = 0; l < 5; ++l) {
    long long v;
    if (std::scanf("%lld", &v) != 1) return 1;
    K.Ml[l] = (double)v;
  }
  for (int l = 0; l < 5; ++l) {
    long long v;
    if (std::scanf("%lld", &v) != 1) return 1;
    K.Hl[l] = (double)v;
  }
  if (std::scanf("%llx %llx", &hb, &ib) != 2) return 1;
  K.halfM = from_bits(hb);
  K.invM = from_bits(ib);
  int count;
  if (std::scanf("%d", &count) != 1) return 1;
  if (W == 40) {
    switch (L) {
      case 1: run<1, 40>(K, count); break;
      case 2: run<2, 40>(K, count); break;
      case 3: run<3, 40>(K, count); break;
    }
    return 0;
  }
  switch (L) {
    case 1: run<1, 32>(K, count); break;
    case 2: run<2, 32>(K, count); break;
    case 3: run<3, 32>(K, count); break;
    case 4: run<4, 32>(K, count); break;
    case 5: run<5, 32>(K, count); break;
    default: return 1;
  }
  return 0;
}
