// CPU emulation of every memory address the product, residue and CRT kernels
// form, for one launch configuration per input line.  It restates the index
// arithmetic of the kernels in csrc/ (gemm_i8.hip, residue.hip, crt.hip,
// accu.hip) on the host, with the grid helpers of csrc/gemm_grid.h itself,
// and checks that every global load and store stays inside its buffer and
// every LDS access inside the block's allocation.
//
// Input lines (all sizes padded as the library pads them):
//   gemm  <form> <m_pad> <n_pad> <q_pad> <s> <cus> <parts> <per> <k_begin> <k_slices> <swz_bug>
//         form: main (residue output, one block per tile), persist (the same,
//         cus blocks walking the tiles), main8 / persist8 (the same with
//         eight wavefronts of 128 x 64), acc (residue output added to the
//         earlier K blocks' residues), ct (int32 output, eight wavefronts),
//         ct4 (int32 output with four wavefronts of 32 x 32 tiles: an earlier
//         form, kept for the planted swizzle case)
//   plan  <m_pad> <n_pad> <q_pad> <nplanes_a> <nplanes_b> then nout lines "a0 b0 count out"
//         (preceded by "<nout>"): int32 output, eight wavefronts
//   reduce <m_pad> <n_pad> <s> <parts>
//   residue <rows> <rows_pad> <q> <q_pad> <s> <rs> <ls> <one_pass>
//   residue_pair <m> <m_pad> <lda> <n> <n_pad> <ldb> <q> <q_pad> <s> <m_stride> <nchunks>
//         (nchunks 0: A's exponents read, not folded)
//   scale_pair <m> <m_pad> <lda> <n> <ldb> <q> <nchunks>
//   crt <m> <n> <m_pad> <n_pad> <s> <ldc>
// Output: one line "ok <accesses>" or "bad <what> ..." per input line.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "../fp64_gemm_emulation_ozii_amd/csrc/gemm_grid.h"

namespace {

long g_checks = 0;
std::string g_bad;

void check(bool ok, const char* what, long a, long b) {
  ++g_checks;
  if (!ok && g_bad.empty()) {
    char buf[256];
    std::snprintf(buf, sizeof buf, "%s %ld %ld", what, a, b);
    g_bad = buf;
  }
}

// [off, off + len) inside [0, size)
void in_range(long off, long len, long size, const char* what) { check(off >= 0 && off + len <= size, what, off, size); }

int swz128(int row, bool bug) { return bug ? (row & 7) : (((row >> 1) ^ (row << 2)) & 7); }

struct Plan {
  int a0, b0, count, out;
};

// The main product kernel: BM = BN = 256, BK = 128 (or 32 with the planted
// swizzle bug), 2 x 2 wavefronts (2 x 4 with `eight`).  MT = 16, except 32
// for int32 output with four wavefronts (the earlier form of `ct4`).
void gemm_main(int m_pad, int n_pad, int q_pad, int s, int cus, bool persist, bool ct, bool acc_rt, int parts,
               int k_begin, int k_slices, bool multi, const std::vector<Plan>& plan, int a_planes, int b_planes,
               bool swz_bug, bool eight = false) {
  const int BM = 256, BN = 256, BK = swz_bug ? 32 : 128, WM = 2, WN = eight ? 4 : 2, NW = WM * WN;
  const int CPR = BK / 16, ROWS_PER_KB = 1024 / BK;
  const int A_LOADS = BM * BK / 1024 / NW, B_LOADS = BN * BK / 1024 / NW, LPW = A_LOADS + B_LOADS;
  const int WTM = BM / WM, WTN = BN / WN;
  const int MT = ct && !eight ? 32 : 16, KSTEP = 1024 / MT, CPS = KSTEP / 16, FM = WTM / MT, FN = WTN / MT;
  const int NKS = BK / KSTEP > 0 ? BK / KSTEP : 1, NF = FM + FN;
  const bool staged = !ct && !acc_rt;  // residue-only output goes through LDS
  const int CS = BM + 16;
  const long OPERANDS = 2L * (BM + BN) * BK;
  const long STAGE_OFF = persist ? (long)(BM + BN) * BK : 0;
  const long SMEM = staged && STAGE_OFF + (long)BN * CS > OPERANDS ? STAGE_OFF + (long)BN * CS : OPERANDS;
  const int tiles_m = m_pad / BM, tiles_n = n_pad / BN, tiles = tiles_m * tiles_n;
  const int nk = q_pad / BK;
  const long a_plane = (long)m_pad * q_pad, b_plane = (long)n_pad * q_pad, plane = (long)m_pad * n_pad;
  const int nplanes = multi ? (int)plan.size() : s * (parts > 1 ? parts : 1);
  const long nblocks = (long)nplanes * tiles;
  const long out_planes = multi ? 0 : nplanes;
  int out_max = 0;
  for (const Plan& p : plan) out_max = p.out + 1 > out_max ? p.out + 1 : out_max;
  const long out_size = (multi ? out_max : out_planes) * plane * (ct ? 4 : 1);
  const long A_size = (long)(multi ? a_planes : s) * a_plane, B_size = (long)(multi ? b_planes : s) * b_plane;
  const long kb_stride = (long)ROWS_PER_KB * q_pad;
  const int grid = persist ? cus : (int)nblocks;
  for (int b = 0; b < grid; ++b) {
    for (long L = b; L < nblocks; L += grid) {
      int tt, mi, nj;
      oz::tile_of_block<4>((int)L, nplanes, tiles_m, tiles_n, tt, mi, nj);
      check(tt >= 0 && tt < nplanes && mi >= 0 && mi < tiles_m && nj >= 0 && nj < tiles_n, "tile", L, nblocks);
      const int m0 = mi * BM, n0 = nj * BN;
      int out_t = tt, part = 0, a0, b0, count = 1;
      if (!multi) {
        part = tt / s;
        tt -= part * s;
        a0 = b0 = tt;
      } else {
        a0 = plan[tt].a0;
        b0 = plan[tt].b0;
        count = plan[tt].count;
        out_t = plan[tt].out;
      }
      const long Ag = (long)a0 * a_plane + (long)m0 * q_pad, Bg = (long)b0 * b_plane + (long)n0 * q_pad;
      const int kfirst = k_begin + part * k_slices;
      const int nkt = multi ? nk * count : (k_slices < nk - kfirst ? k_slices : nk - kfirst);
      check(nkt >= 1, "empty tile", L, nkt);
      for (int kk = 0; kk < nkt; ++kk) {
        long k0 = (long)(kfirst + kk) * BK, ga = Ag, gb = Bg;
        if (multi) {
          const int u = kk / nk;
          k0 = (long)(kk - u * nk) * BK;
          ga += u * a_plane;
          gb -= u * b_plane;
        }
        for (int w = 0; w < NW; ++w)
          for (int li = 0; li < LPW; ++li)
            for (int lane = 0; lane < 64; ++lane) {
              const int lrow = lane / CPR;
              const long src0 = (long)lrow * q_pad + (((lane % CPR) ^ swz128(lrow, swz_bug)) * 16);
              const long src1 = (long)lrow * q_pad + (((lane % CPR) ^ swz128(lrow + ROWS_PER_KB, swz_bug)) * 16);
              const long lds_base = (kk & 1) * (long)(BM + BN) * BK;
              if (li < A_LOADS) {
                const int blk = w * A_LOADS + li;
                in_range(ga + blk * kb_stride + k0 + ((blk & 1) ? src1 : src0), 16, A_size, "gemm A load");
                in_range(lds_base + blk * 1024L + lane * 16, 16, SMEM, "gemm A lds");
              } else {
                const int blk = w * B_LOADS + (li - A_LOADS);
                in_range(gb + blk * kb_stride + k0 + ((blk & 1) ? src1 : src0), 16, B_size, "gemm B load");
                in_range(lds_base + BM * (long)BK + blk * 1024L + lane * 16, 16, SMEM, "gemm B lds");
              }
            }
      }
      // fragment reads (every step of a slice, both buffers)
      if (L == b)
        for (int buf = 0; buf < 2; ++buf)
          for (int ks = 0; ks < NKS; ++ks)
            for (int w = 0; w < NW; ++w)
              for (int f = 0; f < NF; ++f)
                for (int lane = 0; lane < 64; ++lane) {
                  const int wm = w / WN, wn = w % WN, kc = ks * CPS + lane / MT;
                  check(kc < CPR, "fragment chunk", kc, CPR);
                  const long base = buf * (long)(BM + BN) * BK;
                  if (f < FN) {
                    const int row = wn * WTN + f * MT + lane % MT;
                    in_range(base + BM * (long)BK + row * (long)BK + ((kc ^ swz128(row, swz_bug)) * 16), 16, SMEM,
                             "gemm B fragment");
                  } else {
                    const int row = wm * WTM + (f - FN) * MT + lane % MT;
                    in_range(base + row * (long)BK + ((kc ^ swz128(row, swz_bug)) * 16), 16, SMEM, "gemm A fragment");
                  }
                }
      // epilogue
      const long ostride = ct ? 4 : 1;
      for (int w = 0; w < NW; ++w) {
        const int wm = w / WN, wn = w % WN;
        for (int i = 0; i < FM; ++i)
          for (int j = 0; j < FN; ++j)
            for (int lane = 0; lane < 64; ++lane)
              for (int g = 0; g < MT * MT / 64 / 4; ++g) {
                const int lcol = wn * WTN + j * MT + lane % MT;
                const int lrow4 = wm * WTM + i * MT + 8 * g + 4 * (lane / MT);
                const long off = (long)out_t * plane + (long)(n0 + lcol) * m_pad + m0 + lrow4;
                if (staged) {
                  in_range(STAGE_OFF + (long)lcol * CS + lrow4, 4, SMEM, "gemm stage write");
                } else {
                  if (acc_rt) in_range(off, 4, out_size, "gemm residue read");
                  in_range(off * ostride, 4 * ostride, out_size, "gemm direct store");
                }
              }
      }
      if (staged) {
        const int COLS_PER_WAVE = BN / NW, LANES_PER_COL = BM / 16, COLS_PER_STORE = 64 / LANES_PER_COL;
        for (int w = 0; w < NW; ++w)
          for (int it = 0; it < COLS_PER_WAVE / COLS_PER_STORE; ++it)
            for (int lane = 0; lane < 64; ++lane) {
              const int lcol = w * COLS_PER_WAVE + it * COLS_PER_STORE + lane / LANES_PER_COL;
              const int rch = (lane % LANES_PER_COL) * 16;
              in_range(STAGE_OFF + (long)lcol * CS + rch, 16, SMEM, "gemm stage read");
              in_range((long)out_t * plane + (long)(n0 + lcol) * m_pad + m0 + rch, 16, out_size, "gemm staged store");
            }
      }
    }
  }
  check(SMEM <= 160 * 1024, "lds size", SMEM, 160 * 1024);
}

// Sum of the K parts' residues: 16 bytes per thread.
void reduce(int m_pad, int n_pad, int s, int P) {
  const long plane = (long)m_pad * n_pad, chunks = plane / 16, threads = chunks * s;
  for (long gid = 0; gid < (threads + 255) / 256 * 256; gid += 1) {
    if (gid >= chunks * s) continue;
    const long t = gid / chunks, off = (gid - t * chunks) * 16;
    for (int p = 0; p < P; ++p) in_range(((long)p * s + t) * plane + off, 16, (long)P * s * plane, "reduce load");
    in_range(t * plane + off, 16, (long)s * plane, "reduce store");
  }
}

// The residue kernels (and the accu band kernel, the same tile walk): a tile
// of 32 rows x 128 entries per block, 16-byte stores per modulus.
// One 32 x 128 tile (bx, by) of residue_kernel.
void residue_tile(int rows, int rows_pad, int q, int q_pad, int s, long rs, long ls, int bx, int by) {
  const long plane_stride = (long)rows_pad * q_pad;
  const long src_size = rows < 1 ? 0 : (rows - 1) * rs + (q - 1) * ls + 1;
  check(bx >= 0 && bx < q_pad / 128 && by >= 0 && by < rows_pad / 32, "residue tile", bx, by);
        for (int tid = 0; tid < 256; ++tid) {
          const int r0 = by * 32, l0 = bx * 128;
          if (rows >= 1) {
            if (rs == 1) {
              const int r = tid & 31, lsub = tid >> 5;
              for (int it = 0; it < 16; ++it) {
                const long rr = r0 + r < rows - 1 ? r0 + r : rows - 1;
                const long ll = l0 + lsub + 8 * it < q - 1 ? l0 + lsub + 8 * it : q - 1;
                in_range(rr + ll * ls, 1, src_size, "residue load (rows contiguous)");
              }
            } else {
              const int l = tid & 127, rsub = tid >> 7;
              for (int it = 0; it < 16; ++it) {
                const long ll = l0 + l < q - 1 ? l0 + l : q - 1;
                const long rr = r0 + rsub + 2 * it < rows - 1 ? r0 + rsub + 2 * it : rows - 1;
                in_range(ll + rr * rs, 1, src_size, "residue load (inner contiguous)");
              }
            }
          }
          const int r = tid >> 3, cseg = (tid & 7) * 16;
          for (int t = 0; t < s; ++t)
            in_range(t * plane_stride + (long)(r0 + r) * q_pad + l0 + cseg, 16, s * plane_stride, "residue store");
          in_range((long)bx * rows_pad + r0 + r, 1, (long)(q_pad / 128) * rows_pad, "band partial sum");
        }
}

void residue(int rows, int rows_pad, int q, int q_pad, int s, long rs, long ls, bool one_pass) {
  const long plane_stride = (long)rows_pad * q_pad;
  const long src_size = rows < 1 ? 0 : (rows - 1) * rs + (q - 1) * ls + 1;
  if (!one_pass) {
    for (int by = 0; by < rows_pad / 32; ++by)
      for (int bx = 0; bx < q_pad / 128; ++bx) residue_tile(rows, rows_pad, q, q_pad, s, rs, ls, bx, by);
  } else {
    for (int j = 0; j < rows_pad; ++j) {
      if (j < rows)
        for (int l = 0; l < q; ++l) in_range(j * rs + l, 1, src_size, "column residue load");
      for (int seg = 0; seg < q_pad / 16; ++seg)
        for (int t = 0; t < s; ++t)
          in_range(t * plane_stride + (long)j * q_pad + 16L * seg, 16, s * plane_stride, "column residue store");
    }
  }
}

// residue_pair_kernel: blocks [0, na) are column-major A's tiles, the rest
// B's, each decoded from the linear block id over a (q_pad / 128)-wide grid;
// every tile of both grids must come up exactly once.
// With nchunks > 0 (the row-exponent finalisation folded in) every A tile
// also reads its rows' partial row maxima (nchunks words of stride m_stride)
// and the tiles with bx = 0 write the rows' exponents.
void residue_pair(int m, int m_pad, long lda, int n, int n_pad, long ldb, int q, int q_pad, int s, int m_stride,
                  int nchunks) {
  const int gx = q_pad / 128;
  const long na = (long)gx * (m_pad / 32), nb = (long)gx * (n_pad / 32);
  std::vector<int> seen_a(na, 0), seen_b(nb, 0), e_written(m, 0);
  for (long b = 0; b < na + nb; ++b) {
    if (b < na) {
      const int bx = (int)(b % gx), by = (int)(b / gx);
      residue_tile(m, m_pad, q, q_pad, s, 1, lda, bx, by);
      ++seen_a[(long)by * gx + bx];
      if (nchunks > 0)
        for (int tid = 0; tid < 256; ++tid) {
          const int grow = by * 32 + (tid >> 3);
          if (grow >= m) continue;
          for (int cc = tid & 7; cc < nchunks; cc += 8)
            in_range((long)cc * m_stride + grow, 1, (long)nchunks * m_stride, "partial row max load");
          if (bx == 0 && (tid & 7) == 0) {
            in_range(grow, 1, m, "folded exponent store");
            ++e_written[grow];
          }
        }
    } else {
      const int bx = (int)((b - na) % gx), by = (int)((b - na) / gx);
      residue_tile(n, n_pad, q, q_pad, s, ldb, 1, bx, by);
      ++seen_b[(long)by * gx + bx];
    }
  }
  for (long t = 0; t < na; ++t) check(seen_a[t] == 1, "A tile count", t, seen_a[t]);
  for (long t = 0; t < nb; ++t) check(seen_b[t] == 1, "B tile count", t, seen_b[t]);
  if (nchunks > 0)
    for (int i = 0; i < m; ++i) check(e_written[i] == 1, "folded exponent writes", i, e_written[i]);
}

// scale_pair_kernel: blocks [0, na) are row_max_partial_kernel's over a
// (gxa x nchunks) grid, the rest col_exp_kernel's (four columns each).
// fast_pair_kernel (OS II-fast's norm passes) decodes its blocks the same way
// and reads the same elements of A and B.
void scale_pair(int m, int m_pad, long lda, int n, long ldb, int q, int nchunks) {
  const int chunk = (q + nchunks - 1) / nchunks, gxa = (m + 255) / 256;
  const long na = (long)gxa * nchunks, nb = (n + 3) / 4;
  const long a_size = (long)(m - 1) + (long)(q - 1) * lda + 1, b_size = (long)(q - 1) + (long)(n - 1) * ldb + 1;
  std::vector<int> seen(na, 0);
  for (long b = 0; b < na + nb; ++b) {
    if (b < na) {
      const int bx = (int)(b % gxa), by = (int)(b / gxa);
      ++seen[(long)by * gxa + bx];
      for (int tid = 0; tid < 256; ++tid) {
        const int i = bx * 256 + tid, l0 = by * chunk, l1 = q < l0 + chunk ? q : l0 + chunk;
        if (i < m)
          for (int l = l0; l < l1; ++l) in_range(i + (long)l * lda, 1, a_size, "row max load");
        in_range((long)by * m_pad + i, 1, (long)nchunks * m_pad, "row max partial store");
      }
    } else {
      for (int w = 0; w < 4; ++w) {
        const long j = (b - na) * 4 + w;
        if (j >= n) continue;
        for (int l = 0; l < q; ++l) in_range(l + j * ldb, 1, b_size, "column max load");
        in_range(j, 1, n, "column exponent store");
      }
    }
  }
  for (long t = 0; t < na; ++t) check(seen[t] == 1, "row max block count", t, seen[t]);
}

// CRT: four rows of one column per thread, two columns per thread pass.
void crt(int m, int n, int m_pad, int n_pad, int s, long ldc) {
  const long plane = (long)m_pad * n_pad;
  const int NG = (s + 3) / 4;
  // one column per thread for outputs of at most 2^23 entries, else two
  const long cols = (long)m * n <= (1L << 23) ? n : (n + 1) / 2;
  const int gx = (m + 1023) / 1024, gy = (int)(cols < 65535 ? cols : 65535);
  for (int bx = 0; bx < gx; ++bx)
    for (int tx = 0; tx < 256; ++tx) {
      const long i0 = ((long)bx * 256 + tx) * 4;
      if (i0 >= m) continue;
      for (int by = 0; by < gy; ++by)
        for (long j = by; j < n; j += gy) {
          for (int t = 0; t < 4 * NG; ++t)
            if (t < 4 * (NG - 1) || t < s) in_range(j * m_pad + i0 + t * plane, 4, s * plane, "crt load");
          for (int u = 0; u < 4; ++u)
            if (i0 + u < m) in_range(j * ldc + i0 + u, 1, (n - 1) * ldc + m, "crt store");
        }
    }
}

}  // namespace

int main() {
  char cmd[16];
  while (std::scanf("%15s", cmd) == 1) {
    g_checks = 0;
    g_bad.clear();
    if (!std::strcmp(cmd, "gemm")) {
      char form[16];
      int mp, np, qp, s, cus, parts, per, kb, ks, bug;
      if (std::scanf("%15s %d %d %d %d %d %d %d %d %d %d", form, &mp, &np, &qp, &s, &cus, &parts, &per, &kb, &ks,
                     &bug) != 11)
        return 1;
      (void)per;
      const bool eight = !std::strcmp(form, "main8") || !std::strcmp(form, "persist8") || !std::strcmp(form, "ct");
      gemm_main(mp, np, qp, s, cus, !std::strcmp(form, "persist") || !std::strcmp(form, "persist8"),
                !std::strcmp(form, "ct") || !std::strcmp(form, "ct4"), !std::strcmp(form, "acc"), parts, kb, ks, false,
                {}, 0, 0, bug != 0, eight);
    } else if (!std::strcmp(cmd, "plan")) {
      int mp, np, qp, na, nb, nout;
      if (std::scanf("%d %d %d %d %d %d", &mp, &np, &qp, &na, &nb, &nout) != 6) return 1;
      std::vector<Plan> plan(nout);
      for (auto& p : plan)
        if (std::scanf("%d %d %d %d", &p.a0, &p.b0, &p.count, &p.out) != 4) return 1;
      gemm_main(mp, np, qp, 1, 0, false, true, false, 1, 0, qp / 128, true, plan, na, nb, false, true);
    } else if (!std::strcmp(cmd, "reduce")) {
      int mp, np, s, P;
      if (std::scanf("%d %d %d %d", &mp, &np, &s, &P) != 4) return 1;
      reduce(mp, np, s, P);
    } else if (!std::strcmp(cmd, "residue")) {
      int rows, rows_pad, q, q_pad, s, one;
      long rs, ls;
      if (std::scanf("%d %d %d %d %d %ld %ld %d", &rows, &rows_pad, &q, &q_pad, &s, &rs, &ls, &one) != 8) return 1;
      residue(rows, rows_pad, q, q_pad, s, rs, ls, one != 0);
    } else if (!std::strcmp(cmd, "residue_pair")) {
      int m, mp, n, np, q, qp, s, mstride, nch;
      long lda, ldb;
      if (std::scanf("%d %d %ld %d %d %ld %d %d %d %d %d", &m, &mp, &lda, &n, &np, &ldb, &q, &qp, &s, &mstride,
                     &nch) != 11)
        return 1;
      residue_pair(m, mp, lda, n, np, ldb, q, qp, s, mstride, nch);
    } else if (!std::strcmp(cmd, "scale_pair")) {
      int m, mp, n, q, nch;
      long lda, ldb;
      if (std::scanf("%d %d %ld %d %ld %d %d", &m, &mp, &lda, &n, &ldb, &q, &nch) != 7) return 1;
      scale_pair(m, mp, lda, n, ldb, q, nch);
    } else if (!std::strcmp(cmd, "crt")) {
      int m, n, mp, np, s;
      long ldc;
      if (std::scanf("%d %d %d %d %d %ld", &m, &n, &mp, &np, &s, &ldc) != 6) return 1;
      crt(m, n, mp, np, s, ldc);
    } else {
      return 1;
    }
    if (g_bad.empty())
      std::printf("ok %ld\n", g_checks);
    else
      std::printf("bad %s\n", g_bad.c_str());
    std::fflush(stdout);
  }
  return 0;
}
