// Host side of the C-ABI: configuration, argument checks, exact constants
// and the launch sequence of the four steps (Ozaki II notes §7).
#include <hip/hip_runtime.h>

#include <array>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "oz_internal.h"

namespace oz {
namespace {

// ---------------------------------------------------------------------------
// Fixed-width unsigned integers (32-bit limbs, little endian) for the CRT
// constants: M < 2^160 for s <= 20, and Z/2q style divisions by small values.
// ---------------------------------------------------------------------------
constexpr int BIG_LIMBS = 6;
struct Big {
  uint32_t w[BIG_LIMBS] = {0, 0, 0, 0, 0, 0};
};

Big big_from(uint32_t v) {
  Big b;
  b.w[0] = v;
  return b;
}

void big_mul_small(Big& a, uint32_t v) {
  uint64_t carry = 0;
  for (int i = 0; i < BIG_LIMBS; ++i) {
    const uint64_t p = (uint64_t)a.w[i] * v + carry;
    a.w[i] = (uint32_t)p;
    carry = p >> 32;
  }
}

// a / v (v > 0), returns the remainder
uint32_t big_divmod_small(const Big& a, uint32_t v, Big* quot) {
  uint64_t rem = 0;
  Big q;
  for (int i = BIG_LIMBS - 1; i >= 0; --i) {
    const uint64_t cur = (rem << 32) | a.w[i];
    q.w[i] = (uint32_t)(cur / v);
    rem = cur % v;
  }
  if (quot) *quot = q;
  return (uint32_t)rem;
}

void big_sub_small(Big& a, uint32_t v) {
  uint64_t borrow = v;
  for (int i = 0; i < BIG_LIMBS && borrow; ++i) {
    const uint64_t cur = a.w[i];
    a.w[i] = (uint32_t)(cur - borrow);
    borrow = cur < borrow ? 1 : 0;
  }
}

int big_bitlen(const Big& a) {
  for (int i = BIG_LIMBS - 1; i >= 0; --i)
    if (a.w[i]) return 32 * i + (32 - __builtin_clz(a.w[i]));
  return 0;
}

// Bits [lo, lo + width) of a (width <= 40) as a double.
double big_bits(const Big& a, int lo, int width) {
  uint64_t v = 0;
  for (int b = 0; b < width; ++b) {
    const int bit = lo + b;
    if (bit < 32 * BIG_LIMBS && ((a.w[bit / 32] >> (bit % 32)) & 1u)) v |= 1ull << b;
  }
  return (double)v;
}

double big_to_double(const Big& a) {
  double d = 0.0;
  for (int i = BIG_LIMBS - 1; i >= 0; --i) d = d * 4294967296.0 + (double)a.w[i];
  return d;
}

// ---------------------------------------------------------------------------
// Moduli: scan 256 downward, keep each value coprime to all kept ones
// (Ozaki II notes §4 pairwise coprime; §6 m_t <= 256).
// ---------------------------------------------------------------------------
int gcd_int(int a, int b) {
  while (b) {
    const int t = a % b;
    a = b;
    b = t;
  }
  return a;
}

const std::vector<int>& moduli_list() {
  static std::vector<int> mods = [] {
    std::vector<int> out;
    for (int cand = 256; cand >= 2 && (int)out.size() < OZGEMM_S_MAX; --cand) {
      bool ok = true;
      for (int x : out) ok = ok && gcd_int(cand, x) == 1;
      if (ok) out.push_back(cand);
    }
    return out;
  }();
  return mods;
}

Big product_M(int s) {
  Big M = big_from(1);
  for (int t = 0; t < s; ++t) big_mul_small(M, (uint32_t)moduli_list()[t]);
  return M;
}

// k = floor(1/2 floor(log2((M/2 - 1)/q))): largest j with 2q 2^j <= M - 2 is
// bitlen(floor((M - 2) / 2q)) - 1 (Ozaki II notes §5).
int kbits_exact(int s, int q) {
  if (s < 1 || s > OZGEMM_S_MAX || q < 1) return -1;
  Big M = product_M(s);
  big_sub_small(M, 2);
  Big t;
  big_divmod_small(M, 2u * (uint32_t)q, &t);
  const int bl = big_bitlen(t);
  if (bl == 0) return -1;
  return (bl - 1) / 2;
}

// OS II-fast budget (Ozaki II notes §9): kappa_A + kappa_B = floor(log2(M/2 - 1)),
// split evenly, so that ||A'_i|| <= 2^kappa_A and ||B'_j|| <= 2^kappa_B keep
// |(A'B')_ij| < M/2 by Cauchy-Schwarz.
void fast_budget(int s, int* kappa_a, int* kappa_b) {
  Big M = product_M(s);
  Big half;
  big_divmod_small(M, 2, &half);
  big_sub_small(half, 1);
  const int K2 = big_bitlen(half) - 1;
  *kappa_a = K2 / 2;
  *kappa_b = K2 - K2 / 2;
}

// OS II-accu budget constants (Ozaki II notes §9): K2 = floor(log2(M/2 - 1))
// and V = (M/2 - 1) 127^2 2^14, the numerator that the accu kernels compare
// 2^(a_i + b_j) times the two-band bound with: its bit length bv and its top
// 64 bits (bits bv - 64 .. bv - 1).  V < 2^192 for s <= 20.
void accu_budget_consts(int s, int* K2, uint64_t* vtop, int* bv) {
  Big M = product_M(s);
  Big V;
  big_divmod_small(M, 2, &V);
  big_sub_small(V, 1);
  *K2 = big_bitlen(V) - 1;
  big_mul_small(V, 127u * 127u);
  big_mul_small(V, 1u << 14);
  const int b = big_bitlen(V);
  uint64_t top = 0;
  for (int k = 0; k < 64; ++k) {
    const int bit = b - 64 + k;
    if (bit >= 0 && ((V.w[bit / 32] >> (bit % 32)) & 1u)) top |= 1ull << k;
  }
  *bv = b;
  *vtop = top;
}

int modinv_small(int a, int m) {  // a^-1 mod m, gcd(a, m) = 1
  int t = 0, newt = 1, r = m, newr = a % m;
  while (newr) {
    const int qq = r / newr;
    int tmp = t - qq * newt;
    t = newt;
    newt = tmp;
    tmp = r - qq * newr;
    r = newr;
    newr = tmp;
  }
  return t < 0 ? t + m : t;
}

// Shift base k of the residue and CRT kernels and the magnitude bound of A'
// and B' for the active bit budget: the conservative one (k bits, §5) or
// OS II-fast (exponents e' relative to kb = max(kappa_A, kappa_B), §9).
void budget_k(int s, int q, int mode, int* k, int* kmag) {
  if (mode == OZGEMM_BOUND_ACCU) {  // per-row and per-column bit counts up to ACCU_KMAX (§9)
    *k = ACCU_KMAX;
    *kmag = ACCU_KMAX;
  } else if (mode == OZGEMM_BOUND_FAST) {
    int ka, kb;
    fast_budget(s, &ka, &kb);
    *k = std::max(ka, kb);
    *kmag = *k + 1;
  } else {
    *k = kbits_exact(s, q);
    *kmag = *k;
  }
}

// Limb width of the CRT sums: 40 bits while three limbs hold M (log2 M <=
// 120, s <= 15), where r_t w_{t,l} summed over s <= 15 moduli stays below
// 2^53; 32 bits otherwise.
int crt_width(int s) { return big_bitlen(product_M(s)) <= 120 ? 40 : 32; }

void make_consts(int s, int q, int mode, ResidueConsts* rc, GemmConsts* gc, CrtConsts* cc) {
  const auto& mods = moduli_list();
  int k, kmag;
  budget_k(s, q, mode, &k, &kmag);
  std::memset(rc, 0, sizeof(*rc));
  std::memset(gc, 0, sizeof(*gc));
  std::memset(cc, 0, sizeof(*cc));
  rc->s = gc->s = cc->s = s;
  rc->k = cc->k = k;
  rc->kmag = kmag;
  rc->col_kappa = -1;
  if (mode == OZGEMM_BOUND_FAST) {
    int ka = 0, kb = 0;
    fast_budget(s, &ka, &kb);
    rc->col_kappa = kb;  // the columns of B share kappa_B; the shift base k is max(kappa_A, kappa_B)
  }
  for (int t = 0; t < s; ++t) {
    const int m = mods[t];
    rc->m[t] = gc->m[t] = m;
    rc->inv[t] = gc->inv[t] = 1.0 / (double)m;
    rc->c26[t] = (double)((1ull << 26) % (unsigned long long)m);
    rc->c52[t] = (double)((1ull << 52) % (unsigned long long)m);
  }
  const Big M = product_M(s);
  const int bits = big_bitlen(M);
  cc->W = crt_width(s);
  cc->L = (bits + cc->W - 1) / cc->W;
  Big half;
  big_divmod_small(M, 2, &half);
  for (int l = 0; l < MAX_LIMBS; ++l) {
    cc->K.Ml[l] = big_bits(M, l * cc->W, cc->W);
    cc->K.Hl[l] = big_bits(half, l * cc->W, cc->W);
  }
  cc->K.halfM = big_to_double(half);
  cc->K.invM = 1.0 / big_to_double(M);
}

// W_t = M_t y_t limbs (crt_width(s) bits each) for s moduli, written to
// out[t * MAX_LIMBS + l].
void crt_weights(int s, double* out) {
  const auto& mods = moduli_list();
  const Big M = product_M(s);
  const int width = crt_width(s);
  for (int t = 0; t < OZGEMM_S_MAX; ++t)
    for (int l = 0; l < MAX_LIMBS; ++l) out[t * MAX_LIMBS + l] = 0.0;
  for (int t = 0; t < s; ++t) {
    Big Mt;
    const uint32_t mt = (uint32_t)mods[t];
    big_divmod_small(M, mt, &Mt);
    const uint32_t Mt_mod = big_divmod_small(Mt, mt, nullptr);
    const int y = modinv_small((int)Mt_mod, (int)mt);
    Big W = Mt;
    big_mul_small(W, (uint32_t)y);  // W_t = M_t y_t < M
    for (int l = 0; l < MAX_LIMBS; ++l) out[t * MAX_LIMBS + l] = big_bits(W, l * width, width);
  }
}

// ---------------------------------------------------------------------------
// Global configuration and workspace layout
// ---------------------------------------------------------------------------
constexpr int NCH_MAX = 256;  // partial row-max chunks of A
// m x chunks up to which run_dgemm folds the row-exponent finalisation into
// the paired residue pass.  Same-box A/B: 1024^3 (32768) 5% faster per call;
// 2048^3 (131072) no faster, the extra partial reads cost the residue pass
// what the saved launch gains.
constexpr long FOLD_MAX_PARTIALS = 1L << 16;

struct Layout {
  size_t consts, pmax, e, f, ares, bres, rt, rt_bytes, total;
};

Layout make_layout(int max_m, int max_n, int max_q, int s_max, bool split_region = true, size_t rt_min = 0) {
  const size_t mp = round_up((size_t)std::max(max_m, 1), ROW_PAD);
  const size_t np = round_up((size_t)std::max(max_n, 1), ROW_PAD);
  const size_t qp = round_up((size_t)std::max(max_q, 1), K_PAD);
  Layout L;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = round_up(off + bytes, 256);
    return o;
  };
  L.consts = take(CRT_TABLE_DOUBLES * sizeof(double));
  L.pmax = take((size_t)NCH_MAX * mp * 8);
  L.e = take(mp * 4);
  L.f = take(np * 4);
  L.ares = take((size_t)s_max * mp * qp);
  L.bres = take((size_t)s_max * np * qp);
  // product residues; also the K part planes of skinny products (gemm_grid.h)
  L.rt_bytes = std::max({(size_t)s_max * mp * np,
                         split_region ? (size_t)split_region_bytes((int)(qp / K_PAD), ROW_PAD * ROW_PAD) : 0,
                         rt_min});
  L.rt = take(L.rt_bytes);
  L.total = off;
  return L;
}

struct State {
  bool configured = false;
  int s_max = 0, max_m = 0, max_n = 0, max_q = 0;
  hipStream_t stream = nullptr;
  char* ws = nullptr;
  size_t ws_bytes = 0;
  Layout lay{};
  bool consts_on_device = false;  // CRT weight table uploaded to the workspace
  std::vector<double> consts_host;
  int bound = OZGEMM_BOUND_CONSERVATIVE;  // bit budget of Scheme II calls
  bool timing = false;
  std::vector<std::array<hipEvent_t, 5>> events;
  std::string hip_err;
  int panels = 0;  // ozgemm_set_panels: 0 automatic, 1 off, P >= 2 forced
  // the panel pipeline's second stream and its events (created at the first
  // pipelined call, on the device current then)
  hipStream_t side = nullptr;
  std::array<hipEvent_t, OZGEMM_PANELS_MAX + 1> side_ev{};
};
State g;

void release_side() {
  if (g.side != nullptr) {
    (void)hipStreamSynchronize(g.side);
    (void)hipStreamDestroy(g.side);
    for (auto& x : g.side_ev)
      if (x != nullptr) (void)hipEventDestroy(x);
  }
  g.side = nullptr;
  g.side_ev = {};
}

// Where one Scheme II call keeps its intermediates and launches its kernels:
// the configured workspace and stream (ozgemm_dgemm and the stage entry
// points), or the library's fixed device array (ozgemm_dgemm_noalloc).
struct Ctx {
  char* ws;
  Layout lay;
  int row_stride;  // stride of the partial row maxima (rows padded like the layout's largest m)
  hipStream_t stream;
  int bound;
  int panels = 1;                // column panels of the pipeline (1: none)
  hipStream_t side = nullptr;    // the pipeline's second stream
  const hipEvent_t* side_ev = nullptr;
};

Ctx config_ctx() {
  return Ctx{g.ws, g.lay, (int)round_up((size_t)std::max(g.max_m, 1), ROW_PAD), g.stream, g.bound};
}

constexpr size_t TIMING_MAX_CALLS = 4096;
// the residue and Scheme I split grids index tiles of 32 rows in grid.y
// (<= 65535), over rows padded to ROW_PAD
constexpr int OZ_MAX_ROWS = OZGEMM_MAX_ROWS;
static_assert((OZ_MAX_ROWS + ROW_PAD - 1) / ROW_PAD * ROW_PAD / 32 <= 65535, "row tiles fit grid.y");

int hip_fail(hipError_t err) {
  g.hip_err = hipGetErrorString(err);
  return OZGEMM_HIP_ERROR;
}

#define OZ_CHECK(expr)                             \
  do {                                             \
    const hipError_t oz_err_ = (expr);             \
    if (oz_err_ != hipSuccess) return hip_fail(oz_err_); \
  } while (0)

// Compute units of the current device (queried once per device).
int device_cus(int* cus) {
  constexpr int MAX_DEVICES = 64;
  static int cached[MAX_DEVICES] = {};
  int dev = 0;
  OZ_CHECK(hipGetDevice(&dev));
  if (dev < 0 || dev >= MAX_DEVICES) return hip_fail(hipErrorInvalidDevice);
  if (cached[dev] == 0) {
    int v = 0;
    OZ_CHECK(hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev));
    cached[dev] = std::max(v, 1);
  }
  *cus = cached[dev];
  return 0;
}

// K parts of a residue-only Scheme II product of padded size mp x np x qp
// (gemm_grid.h); their planes go to the workspace's product region.
int product_split(const Layout& lay, int mp, int np, int qp, int s, SplitChoice* out, int* cus) {
  const int st = device_cus(cus);
  if (st) return st;
  const long cap = (long)(lay.rt_bytes / ((size_t)mp * np));
  *out = choose_splits((mp / ROW_PAD) * (np / ROW_PAD), s, qp / K_PAD, *cus, cap);
  return 0;
}

// The CRT weight table lives in the workspace; it is copied there once after
// each configuration, at the first call that needs it (a blocking 16 KB copy).
int ensure_crt_table() {
  if (g.consts_on_device) return 0;
  g.consts_host.assign(CRT_TABLE_DOUBLES, 0.0);
  for (int s = 1; s <= OZGEMM_S_MAX; ++s) crt_weights(s, g.consts_host.data() + (size_t)(s - 1) * OZGEMM_S_MAX * MAX_LIMBS);
  OZ_CHECK(hipMemcpy(g.ws + g.lay.consts, g.consts_host.data(), CRT_TABLE_DOUBLES * sizeof(double),
                     hipMemcpyHostToDevice));
  g.consts_on_device = true;
  return 0;
}

const double* crt_table(int s) {
  return reinterpret_cast<const double*>(g.ws + g.lay.consts) + (size_t)(s - 1) * OZGEMM_S_MAX * MAX_LIMBS;
}

void dims(int m, int n, int q, int* mp, int* np, int* qp) {
  *mp = (int)round_up((size_t)std::max(m, 1), ROW_PAD);
  *np = (int)round_up((size_t)std::max(n, 1), ROW_PAD);
  *qp = (int)round_up((size_t)std::max(q, 1), K_PAD);
}

bool overlaps(const void* a, size_t abytes, const void* b, size_t bbytes) {
  const char* pa = (const char*)a;
  const char* pb = (const char*)b;
  return pa < pb + bbytes && pb < pa + abytes;
}

size_t mat_bytes(int rows, int cols, int ld) {
  if (rows == 0 || cols == 0) return 0;
  return ((size_t)ld * (size_t)(cols - 1) + (size_t)rows) * sizeof(double);
}

// Shared checks of (m, n, q, A, lda, B, ldb) and the size/range limits.
int check_common(int m, int n, int q, const double* A, int lda, const double* B, int ldb) {
  if (m < 0) return -1;
  if (n < 0) return -2;
  if (q < 0) return -3;
  if (A == nullptr && m > 0 && q > 0) return -4;
  if (lda < std::max(1, m)) return -5;
  if (B == nullptr && q > 0 && n > 0) return -6;
  if (ldb < std::max(1, q)) return -7;
  return 0;
}

// Limits of the method and of the active bit budget (any entry point).
int check_method_range(int q, int s) {
  if (q > OZGEMM_Q_MAX) return OZGEMM_RANGE;
  if (g.bound != OZGEMM_BOUND_FAST && q > 0 && kbits_exact(s, q) < 1) return OZGEMM_RANGE;
  if (g.bound == OZGEMM_BOUND_FAST && q >= OZGEMM_FAST_Q_LIMIT) return OZGEMM_RANGE;  // 64-bit norm sums
  if (g.bound == OZGEMM_BOUND_ACCU && (q > OZGEMM_ACCU_Q_MAX || s < 2)) return OZGEMM_RANGE;
  return 0;
}

int check_range(int m, int n, int q, int s) {
  if (!g.configured) return OZGEMM_NOT_CONFIGURED;
  if (m > g.max_m || n > g.max_n || q > g.max_q || s > g.s_max) return OZGEMM_RANGE;
  return check_method_range(q, s);
}

int nchunks_for(int m, int q) {
  const int xblocks = (m + 255) / 256;
  int nch = (4096 + xblocks - 1) / xblocks;
  nch = std::min(nch, (q + 31) / 32);
  nch = std::min(nch, NCH_MAX);
  return std::max(nch, 1);
}

// Room for OS II-accu's intermediates: the band planes use the residue
// regions, the bound's int32 and L planes the product region, the partial
// row sums of A's low band the partial row-max region; all of it is dead
// until the residue step.
bool accu_fits(const Layout& lay, int m, int n, int q) {
  if (m < 1 || n < 1 || q < 1) return true;
  int mpc, npc, qpc;
  dims(m, n, q, &mpc, &npc, &qpc);
  return lay.bres - lay.ares >= 2 * (size_t)mpc * qpc && lay.rt - lay.bres >= 2 * (size_t)npc * qpc &&
         lay.rt_bytes >= accu_scratch_bytes(mpc, npc, qpc) && (size_t)qpc / K_PAD * 4 <= (size_t)NCH_MAX * 8;
}

// With fold_e (conservative budget, both operands) A's row exponents are
// left to the paired residue pass, which reduces the partial row maxima
// itself (launch_residue_pair with pmax).
int run_scale(const Ctx& x, int m, int n, int q, int s, const double* A, int lda, const double* B, int ldb,
              int32_t* e, int32_t* f, bool fold_e = false) {
  const int mp = x.row_stride;
  uint64_t* pmax = reinterpret_cast<uint64_t*>(x.ws + x.lay.pmax);
  const int nch = nchunks_for(m, q);
  const bool fast = x.bound == OZGEMM_BOUND_FAST;
  int ka = 0, kb = 0;
  if (fast) fast_budget(s, &ka, &kb);
  const int kbase = std::max(ka, kb);
  if (m > 0 && n > 0 && q > 0) {
    // A's partial row maxima and B's column maxima in one launch
    OZ_CHECK(launch_scale_pair(A, m, q, lda, pmax, mp, nch, B, n, ldb, f, x.stream));
    if (!fold_e) OZ_CHECK(launch_row_exp_finalize(pmax, m, mp, nch, e, x.stream));
    if (fast) OZ_CHECK(launch_fast_pair(A, m, q, lda, pmax, mp, nch, ka, B, n, ldb, kb, kbase, e, f, x.stream));
  } else {
    if (m > 0) {
      OZ_CHECK(launch_row_max_partial(A, m, q, lda, pmax, mp, nch, x.stream));
      OZ_CHECK(launch_row_exp_finalize(pmax, m, mp, nch, e, x.stream));
      if (fast) OZ_CHECK(launch_row_fast(A, m, q, lda, pmax, mp, nch, ka, kbase, e, x.stream));
    }
    if (n > 0) {
      OZ_CHECK(launch_col_exp(B, q, n, ldb, f, x.stream));
      if (fast) OZ_CHECK(launch_col_fast(B, q, n, ldb, kb, kbase, f, x.stream));
    }
  }
  if (x.bound == OZGEMM_BOUND_ACCU && m > 0 && n > 0 && q > 0) {
    int mpc, npc, qpc;
    dims(m, n, q, &mpc, &npc, &qpc);
    if (!accu_fits(x.lay, m, n, q)) return OZGEMM_WORKSPACE_TOO_SMALL;  // checked before any launch by callers
    int K2 = 0, bv = 0;
    uint64_t vtop = 0;
    accu_budget_consts(s, &K2, &vtop, &bv);
    OZ_CHECK(launch_accu_exponents(A, m, q, lda, B, n, ldb, mpc, npc, qpc, K2, vtop, bv, ACCU_KMAX,
                                   reinterpret_cast<int8_t*>(x.ws + x.lay.ares),
                                   reinterpret_cast<int8_t*>(x.ws + x.lay.bres), reinterpret_cast<int32_t*>(pmax),
                                   x.ws + x.lay.rt, e, f, x.stream));
  }
  return 0;
}

int run_residue(int m, int n, int q, int s, const double* A, int lda, const double* B, int ldb, const int32_t* e,
                const int32_t* f, int8_t* Ares, int8_t* Bres, double* Ap, double* Bp) {
  int mp, np, qp;
  dims(m, n, q, &mp, &np, &qp);
  ResidueConsts rc;
  GemmConsts gc;
  CrtConsts cc;
  make_consts(s, q, g.bound, &rc, &gc, &cc);
  // A: element (i, l) at A[i + l*lda]; A' copy m x q with ld m
  OZ_CHECK(launch_residue(A, m, q, 1, lda, e, rc, Ares, mp, qp, Ap, 1, m, g.stream));
  // B seen as rows j: element (j, l) at B[l + j*ldb]; B' copy q x n with ld q
  OZ_CHECK(launch_residue(B, n, q, ldb, 1, f, rc, Bres, np, qp, Bp, q, 1, g.stream));
  return 0;
}

// ---------------------------------------------------------------------------
// Scheme I (slice split) helpers
// ---------------------------------------------------------------------------

// beta = min(7, floor((31 - log2 q) / 2)) as the largest b <= 7 with
// q 4^b <= 2^31 (Ozaki I notes, RN split analysis); -1 when no b >= 1 fits.
int s1_beta(int q) {
  if (q < 1) return -1;
  int b = 0;
  while (b < 7 && (int64_t)q * ((int64_t)1 << (2 * (b + 1))) <= ((int64_t)1 << 31)) ++b;
  return b >= 1 ? b : -1;
}

// r = max(1, 2^(31 - 2 beta - ceil(log2 q))) (Ozaki I notes, direction 2).
int s1_group(int q, int beta) {
  const int c = (q <= 1) ? 0 : 32 - __builtin_clz((unsigned)(q - 1));
  const int e = 31 - 2 * beta - c;
  return e >= 0 ? std::max(1, 1 << e) : 1;
}

int s1_nout(int k, int variant, int r) {
  if (variant == OZGEMM_S1_RN) return k * (k + 1) / 2;
  int total = 0;
  for (int gg = 2; gg <= k + 1; ++gg) total += (gg - 1 + r - 1) / r;
  return total;
}

struct S1Layout {
  size_t plans, gA, gB, pmax, asl, bsl, P, total;  // offsets from the Scheme I base
  int mp, np, qp, grid_rows, nout, nch, beta, r;
};

S1Layout s1_layout(int m, int n, int q, int k, int variant) {
  S1Layout L{};
  dims(m, n, q, &L.mp, &L.np, &L.qp);
  L.beta = s1_beta(std::max(q, 1));
  L.r = s1_group(std::max(q, 1), std::max(L.beta, 1));
  L.grid_rows = variant == OZGEMM_S1_RN ? k : 1;
  L.nout = s1_nout(k, variant, L.r);
  L.nch = L.qp / 128;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = round_up(off + bytes, 256);
    return o;
  };
  L.plans = take(2 * OZGEMM_S1_MAX_OUT * sizeof(int4));
  L.gA = take((size_t)L.grid_rows * L.mp * 4);
  L.gB = take((size_t)L.grid_rows * L.np * 4);
  L.pmax = take((size_t)L.nch * std::max(L.mp, L.np) * 8);
  L.asl = take((size_t)k * L.mp * L.qp);
  L.bsl = take((size_t)k * L.np * L.qp);
  L.P = take((size_t)L.nout * L.mp * L.np * 4);
  L.total = off;
  return L;
}

// Scheme I scratch starts after the constant table shared with Scheme II.
size_t s1_base() { return round_up(CRT_TABLE_DOUBLES * sizeof(double), 256); }

int s1_check(int k, int variant, int q) {
  if (k < 1 || k > OZGEMM_S1_K_MAX) return -1;
  if (variant != OZGEMM_S1_RN && variant != OZGEMM_S1_HYBRID) return -2;
  if (q > 0 && s1_beta(q) < 1) return OZGEMM_RANGE;
  return 0;
}

// Split of A (rows) and B (columns) into slices and grid exponents.
int s1_split(const S1Layout& L, int m, int n, int q, int k, int variant, const double* A, int lda, const double* B,
             int ldb, int8_t* Asl, int8_t* Bsl, int32_t* gA, int32_t* gB, uint64_t* pmax) {
  struct Side {
    const double* X;
    int rows;
    long rs, ls;
    int rp;
    int8_t* sl;
    int32_t* gr;
  } sides[2] = {{A, m, 1, (long)lda, L.mp, Asl, gA}, {B, n, (long)ldb, 1, L.np, Bsl, gB}};
  for (const Side& sd : sides) {
    if (sd.ls == 1 && s1_row_split_fits(q)) {  // rows contiguous and short enough to hold: one pass
      OZ_CHECK(launch_s1_row_split(sd.X, sd.rows, q, sd.rs, sd.rp, L.qp, variant, k, L.beta, sd.gr, sd.sl,
                                   g.stream));
      continue;
    }
    OZ_CHECK(launch_s1_rowmax(sd.X, sd.rows, q, sd.rs, sd.ls, sd.rp, L.qp, pmax, g.stream));
    OZ_CHECK(launch_s1_grid(pmax, sd.rp, L.nch, L.beta, sd.gr, g.stream));
    if (variant == OZGEMM_S1_RN) {
      for (int p = 0; p < k; ++p) {
        const bool more = p + 1 < k;
        OZ_CHECK(launch_s1_split(sd.X, sd.rows, q, sd.rs, sd.ls, sd.gr, sd.rp, L.qp, variant, p, k, L.beta, sd.sl,
                                 more ? pmax : nullptr, g.stream));
        if (more) OZ_CHECK(launch_s1_grid(pmax, sd.rp, L.nch, L.beta, sd.gr + (size_t)(p + 1) * sd.rp, g.stream));
      }
    } else {
      OZ_CHECK(launch_s1_split(sd.X, sd.rows, q, sd.rs, sd.ls, sd.gr, sd.rp, L.qp, variant, 0, k, L.beta, sd.sl,
                               nullptr, g.stream));
    }
  }
  return 0;
}

// Phase-timing events only carry timestamps, read after the caller has
// synchronised, so they skip the system-scope release a default event record
// performs: that fence (a cache write-back between dependent kernels) cost
// about 6 us per record, 18 us per timed call (1024^3: 83 against 65 us
// untimed; 74 us without the fence).
constexpr unsigned kTimingEventFlags = hipEventDisableSystemFence;

// Argument checks of ozgemm_dgemm and ozgemm_dgemm_noalloc (BLAS style).
int check_dgemm_args(int m, int n, int q, const double* A, int lda, const double* B, int ldb, const double* C,
                     int ldc, int s) {
  const int st = check_common(m, n, q, A, lda, B, ldb);
  if (st) return st;
  if (C == nullptr && m > 0 && n > 0) return -8;
  if (ldc < std::max(1, m)) return -9;
  if (s < 1 || s > OZGEMM_S_MAX) return -10;
  if (m > 0 && n > 0) {
    const size_t cb = mat_bytes(m, n, ldc);
    if (overlaps(C, cb, A, mat_bytes(m, q, lda)) || overlaps(C, cb, B, mat_bytes(q, n, ldb))) return -8;
  }
  return 0;
}

// Column panels for the pipeline of an m_pad x n_pad x q_pad product with
// s moduli (1: no pipeline).  Only when asked for (ozgemm_set_panels): on
// MI355X the persistent product grid holds every compute unit (456 of a
// SIMD's 512 registers), so a panel's CRT runs only in the gaps between
// product blocks, and the pipelined call measured 1.5-2% slower than the
// plain one at 16384 x 16384 x 1024 and 8192^3.  Each panel's product is
// one launch of one K part (parts would overwrite the other panels'
// residues).
int choose_panels(int mp, int np, int qp, int s, int cus) {
  if (g.panels < 2 || qp >= OZGEMM_Q_LIMIT) return 1;
  int P = std::min({g.panels, np / ROW_PAD, OZGEMM_PANELS_MAX});
  if (P < 2) return 1;
  const int npp = (int)round_up((size_t)((np + P - 1) / P), ROW_PAD);
  P = (np + npp - 1) / npp;
  const int tiles = (mp / ROW_PAD) * (npp / ROW_PAD);
  if (P < 2 || choose_splits(tiles, s, qp / K_PAD, cus, s).parts != 1) return 1;
  return P;
}

int ensure_side() {
  if (g.side != nullptr) return 0;
  OZ_CHECK(hipStreamCreateWithFlags(&g.side, hipStreamNonBlocking));
  for (auto& x : g.side_ev) {
    const hipError_t err = hipEventCreateWithFlags(&x, hipEventDisableTiming);
    if (err != hipSuccess) {
      x = nullptr;
      release_side();  // all or nothing: the next pipelined call starts over
      return hip_fail(err);
    }
  }
  return 0;
}

// The four steps of one Scheme II call (Ozaki II notes §7) on the buffers of
// x: scale, residues, the int8 products with their reduction mod m_t, and the
// CRT with unscaling.  wtab is the device table of the W_t limbs for s.
// With ev, HIP events are recorded around the phases.
int run_dgemm(const Ctx& x, const double* wtab, int m, int n, int q, const double* A, int lda, const double* B,
              int ldb, double* C, int ldc, int s, std::array<hipEvent_t, 5>* ev) {
  if (q == 0) {
    OZ_CHECK(launch_fill_zero(C, m, n, ldc, x.stream));
    return OZGEMM_OK;
  }
  int mp, np, qp;
  dims(m, n, q, &mp, &np, &qp);
  int32_t* e = reinterpret_cast<int32_t*>(x.ws + x.lay.e);
  int32_t* f = reinterpret_cast<int32_t*>(x.ws + x.lay.f);
  int8_t* Ares = reinterpret_cast<int8_t*>(x.ws + x.lay.ares);
  int8_t* Bres = reinterpret_cast<int8_t*>(x.ws + x.lay.bres);
  uint8_t* rt = reinterpret_cast<uint8_t*>(x.ws + x.lay.rt);

  ResidueConsts rc;
  GemmConsts gc;
  CrtConsts cc;
  make_consts(s, q, x.bound, &rc, &gc, &cc);
  cc.wtab = wtab;
  int st = 0;
  if (ev) OZ_CHECK(hipEventRecord((*ev)[0], x.stream));
  // B's exponents come out of its residue pass when the column fits (under
  // OS II-fast with the column's norm bound too); OS II-accu needs them
  // before its bound, so it keeps two passes
  const bool b_one_pass = x.bound != OZGEMM_BOUND_ACCU && col_residue_fits(q);
  // Small products under the conservative budget skip the row-exponent
  // finalisation launch: the paired residue pass reduces the partial row
  // maxima itself (every A tile re-reads its rows' partials, so only while
  // they are few).
  const int nch = nchunks_for(m, q);
  const bool fold_e = x.bound == OZGEMM_BOUND_CONSERVATIVE && !b_one_pass && x.panels <= 1 &&
                      (long)m * nch <= FOLD_MAX_PARTIALS;
  if ((st = run_scale(x, m, b_one_pass ? 0 : n, q, s, A, lda, B, ldb, e, f, fold_e))) return st;
  if (ev) OZ_CHECK(hipEventRecord((*ev)[1], x.stream));
  if (x.panels > 1) {
    OZ_CHECK(launch_residue(A, m, q, 1, lda, e, rc, Ares, mp, qp, nullptr, 0, 0, x.stream));
    // Panel pipeline (Ozaki II notes §8 and §11: the CRT of one part of C
    // runs while the products of the next part do).  Column panel p of C
    // keeps its B residue planes and product residues contiguous (planes of
    // its own width), so each panel is an ordinary product launch; its CRT
    // goes on the second stream, ordered by an event, while the next
    // panel's product runs.  The call's stream waits for the last CRT.
    if (ev) OZ_CHECK(hipEventRecord((*ev)[2], x.stream));
    int cus = 0;
    if ((st = device_cus(&cus))) return st;
    const int npp = (int)round_up((size_t)((np + x.panels - 1) / x.panels), ROW_PAD);
    for (int j0 = 0, p = 0; j0 < n; j0 += npp, ++p) {
      const int w = std::min(npp, np - j0);          // padded width of this panel
      const int cols = std::min(npp, n - j0);        // its columns of C
      int8_t* Bp = Bres + (size_t)s * qp * j0;
      uint8_t* rp = rt + (size_t)s * mp * j0;
      if (b_one_pass)
        OZ_CHECK(launch_col_residue(B + (size_t)j0 * ldb, cols, q, ldb, f + j0, rc, Bp, w, qp, x.stream));
      else
        OZ_CHECK(launch_residue(B + (size_t)j0 * ldb, cols, q, ldb, 1, f + j0, rc, Bp, w, qp, nullptr, 0, 0,
                                x.stream));
      OZ_CHECK(launch_gemm(Ares, Bp, mp, w, qp, gc, nullptr, rp, SplitChoice{1, qp / K_PAD}, rp, cus, x.stream));
      OZ_CHECK(hipEventRecord(x.side_ev[p], x.stream));
      OZ_CHECK(hipStreamWaitEvent(x.side, x.side_ev[p], 0));
      OZ_CHECK(launch_crt(rp, m, cols, mp, w, e, f + j0, cc, C + (size_t)j0 * ldc, ldc, x.side));
    }
    if (ev) OZ_CHECK(hipEventRecord((*ev)[3], x.stream));
    OZ_CHECK(hipEventRecord(x.side_ev[OZGEMM_PANELS_MAX], x.side));
    OZ_CHECK(hipStreamWaitEvent(x.stream, x.side_ev[OZGEMM_PANELS_MAX], 0));
    if (ev) OZ_CHECK(hipEventRecord((*ev)[4], x.stream));
    return OZGEMM_OK;
  }
  if (b_one_pass) {
    OZ_CHECK(launch_residue(A, m, q, 1, lda, e, rc, Ares, mp, qp, nullptr, 0, 0, x.stream));
    OZ_CHECK(launch_col_residue(B, n, q, ldb, f, rc, Bres, np, qp, x.stream));
  } else if (fold_e) {  // A's and B's residues in one launch, A's exponents from the partial maxima
    OZ_CHECK(launch_residue_pair(A, m, lda, e, Ares, mp, B, n, ldb, f, Bres, np, q, qp, rc, x.stream,
                                 reinterpret_cast<const uint64_t*>(x.ws + x.lay.pmax), x.row_stride, nch));
  } else {  // A's and B's residues in one launch
    OZ_CHECK(launch_residue_pair(A, m, lda, e, Ares, mp, B, n, ldb, f, Bres, np, q, qp, rc, x.stream));
  }
  if (ev) OZ_CHECK(hipEventRecord((*ev)[2], x.stream));
  SplitChoice split{};
  int cus = 0;
  if ((st = product_split(x.lay, mp, np, qp, s, &split, &cus))) return st;
  OZ_CHECK(launch_gemm(Ares, Bres, mp, np, qp, gc, nullptr, rt, split, rt, cus, x.stream));
  if (ev) OZ_CHECK(hipEventRecord((*ev)[3], x.stream));
  OZ_CHECK(launch_crt(rt, m, n, mp, np, e, f, cc, C, ldc, x.stream));
  if (ev) OZ_CHECK(hipEventRecord((*ev)[4], x.stream));
  return OZGEMM_OK;
}

// ---------------------------------------------------------------------------
// The fixed device array of ozgemm_dgemm_noalloc.  Host code never uses the
// array's name as an address: the device address of each GPU's copy comes
// from hipGetSymbolAddress, once per device, and is kept here.  The first
// call on a device also copies the CRT weight table into the array's head.
// ---------------------------------------------------------------------------
static __device__ __align__(256) char scratch[OZGEMM_NOALLOC_BYTES];

int noalloc_scratch(char** out) {
  constexpr int MAX_DEVICES = 64;
  static char* ptr[MAX_DEVICES] = {};
  int dev = 0;
  OZ_CHECK(hipGetDevice(&dev));
  if (dev < 0 || dev >= MAX_DEVICES) return hip_fail(hipErrorInvalidDevice);
  if (ptr[dev] == nullptr) {
    void* p = nullptr;
    OZ_CHECK(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (p == nullptr) return hip_fail(hipErrorInvalidSymbol);
    std::vector<double> table(CRT_TABLE_DOUBLES, 0.0);
    for (int s = 1; s <= OZGEMM_S_MAX; ++s) crt_weights(s, table.data() + (size_t)(s - 1) * OZGEMM_S_MAX * MAX_LIMBS);
    // the table sits at offset 0 of every layout (Layout::consts)
    OZ_CHECK(hipMemcpy(p, table.data(), CRT_TABLE_DOUBLES * sizeof(double), hipMemcpyHostToDevice));
    ptr[dev] = static_cast<char*>(p);
  }
  *out = ptr[dev];
  return 0;
}

}  // namespace
}  // namespace oz

using namespace oz;

extern "C" {

size_t ozgemm_workspace_bytes(int max_m, int max_n, int max_q, int s_max) {
  if (max_m < 0 || max_n < 0 || max_q < 0 || s_max < 1 || s_max > OZGEMM_S_MAX) return 0;
  return make_layout(max_m, max_n, max_q, s_max).total;
}

int ozgemm_config(int s_max, int max_m, int max_n, int max_q, void* hip_stream, void* workspace,
                  size_t workspace_bytes) {
  if (s_max < 1 || s_max > OZGEMM_S_MAX) return -1;
  if (max_m < 0 || max_m > OZ_MAX_ROWS) return -2;
  if (max_n < 0 || max_n > OZ_MAX_ROWS) return -3;
  if (max_q < 0 || max_q > OZGEMM_Q_MAX) return -4;
  if (workspace == nullptr) return -6;
  const Layout lay = make_layout(max_m, max_n, max_q, s_max);
  if (workspace_bytes < lay.total) return OZGEMM_WORKSPACE_TOO_SMALL;
  ozgemm_timing(0);
  release_side();  // the next pipelined call creates it on the device current then
  g.configured = true;
  g.s_max = s_max;
  g.max_m = max_m;
  g.max_n = max_n;
  g.max_q = max_q;
  g.stream = (hipStream_t)hip_stream;
  g.ws = (char*)workspace;
  g.ws_bytes = workspace_bytes;
  g.lay = lay;
  g.consts_on_device = false;
  return OZGEMM_OK;
}

int ozgemm_set_stream(void* hip_stream) {
  if (!g.configured) return OZGEMM_NOT_CONFIGURED;
  g.stream = (hipStream_t)hip_stream;
  return OZGEMM_OK;
}

int ozgemm_free(void) {
  ozgemm_timing(0);
  release_side();
  g = State{};
  return OZGEMM_OK;
}

int ozgemm_set_panels(int panels) {
  if (panels < 0 || panels > OZGEMM_PANELS_MAX) return -1;
  g.panels = panels;
  return OZGEMM_OK;
}

const char* ozgemm_strerror(int status) {
  static thread_local std::string msg;
  if (status == OZGEMM_OK) return "success";
  if (status < 0) {
    msg = "invalid argument " + std::to_string(-status);
    return msg.c_str();
  }
  switch (status) {
    case OZGEMM_NOT_CONFIGURED: return "ozgemm_config has not been called";
    case OZGEMM_RANGE:
      return "problem outside the supported range (q > 2^27, k < 1 under the conservative budget, q >= 2^23 under "
             "OS II-fast, int32 product planes asked for at q >= 2^17, or a size above the configured maximum)";
    case OZGEMM_WORKSPACE_TOO_SMALL: return "workspace smaller than ozgemm_workspace_bytes";
    case OZGEMM_HIP_ERROR:
      msg = "HIP error: " + g.hip_err;
      return msg.c_str();
    default: return "unknown status";
  }
}

int ozgemm_moduli(int s, int* moduli_out) {
  if (s < 1 || s > OZGEMM_S_MAX || moduli_out == nullptr) return -1;
  for (int t = 0; t < s; ++t) moduli_out[t] = moduli_list()[t];
  return 0;
}

int ozgemm_kbits(int s, int q) {
  if (q > OZGEMM_Q_MAX) return -2;
  return kbits_exact(s, q);
}

int ozgemm_plane_dims(int m, int n, int q, int* m_pad, int* n_pad, int* q_pad) {
  if (m < 0 || n < 0 || q < 0 || !m_pad || !n_pad || !q_pad) return -1;
  dims(m, n, q, m_pad, n_pad, q_pad);
  return 0;
}

int ozgemm_dgemm(int m, int n, int q, const double* A, int lda, const double* B, int ldb, double* C, int ldc,
                 int s) {
  int st = check_dgemm_args(m, n, q, A, lda, B, ldb, C, ldc, s);
  if (st) return st;
  if ((st = check_range(m, n, q, s))) return st;
  if (m == 0 || n == 0) return OZGEMM_OK;
  if (g.bound == OZGEMM_BOUND_ACCU && !accu_fits(g.lay, m, n, q)) return OZGEMM_WORKSPACE_TOO_SMALL;
  if ((st = ensure_crt_table())) return st;
  std::array<hipEvent_t, 5> ev{};
  const bool timed = g.timing && g.events.size() < TIMING_MAX_CALLS;
  if (timed)
    for (auto& x : ev) OZ_CHECK(hipEventCreateWithFlags(&x, kTimingEventFlags));
  Ctx x = config_ctx();
  if (q > 0) {
    int mp, np, qp, cus = 0;
    dims(m, n, q, &mp, &np, &qp);
    if ((st = device_cus(&cus))) return st;
    x.panels = choose_panels(mp, np, qp, s, cus);
    if (x.panels > 1) {
      if ((st = ensure_side())) return st;
      x.side = g.side;
      x.side_ev = g.side_ev.data();
    }
  }
  st = run_dgemm(x, crt_table(s), m, n, q, A, lda, B, ldb, C, ldc, s, timed ? &ev : nullptr);
  if (timed) {
    if (st == OZGEMM_OK)
      g.events.push_back(ev);
    else
      for (auto& h : ev) (void)hipEventDestroy(h);
  }
  return st;
}

int ozgemm_dgemm_noalloc(int m, int n, int q, const double* A, int lda, const double* B, int ldb, double* C,
                         int ldc, int s, void* hip_stream) {
  int st = check_dgemm_args(m, n, q, A, lda, B, ldb, C, ldc, s);
  if (st) return st;
  if (m > OZ_MAX_ROWS || n > OZ_MAX_ROWS || (st = check_method_range(q, s))) return OZGEMM_RANGE;
  size_t rt_min = 0;
  if (g.bound == OZGEMM_BOUND_ACCU) {
    int mp0, np0, qp0;
    dims(m, n, q, &mp0, &np0, &qp0);
    rt_min = accu_scratch_bytes(mp0, np0, qp0);
  }
  const Layout lay = make_layout(m, n, q, s, false, rt_min);
  if (lay.total > OZGEMM_NOALLOC_BYTES) return OZGEMM_RANGE;
  if (g.bound == OZGEMM_BOUND_ACCU && !accu_fits(lay, m, n, q)) return OZGEMM_RANGE;
  if (m == 0 || n == 0) return OZGEMM_OK;
  char* base = nullptr;
  if ((st = noalloc_scratch(&base))) return st;
  int mp, np, qp;
  dims(m, n, q, &mp, &np, &qp);
  const Ctx x{base, lay, mp, (hipStream_t)hip_stream, g.bound};
  return run_dgemm(x, reinterpret_cast<const double*>(base + lay.consts) + (size_t)(s - 1) * OZGEMM_S_MAX * MAX_LIMBS,
                   m, n, q, A, lda, B, ldb, C, ldc, s, nullptr);
}

int ozgemm_stage_scale(int m, int n, int q, int s, const double* A, int lda, const double* B, int ldb, int32_t* e,
                       int32_t* f) {
  if (m < 0) return -1;
  if (n < 0) return -2;
  if (q < 0) return -3;
  if (s < 1 || s > OZGEMM_S_MAX) return -4;
  if (A == nullptr && m > 0 && q > 0) return -5;
  if (lda < std::max(1, m)) return -6;
  if (B == nullptr && q > 0 && n > 0) return -7;
  if (ldb < std::max(1, q)) return -8;
  if (e == nullptr && m > 0) return -9;
  if (f == nullptr && n > 0) return -10;
  if (!g.configured) return OZGEMM_NOT_CONFIGURED;
  if (m > g.max_m || n > g.max_n || q > g.max_q || s > g.s_max) return OZGEMM_RANGE;
  if (g.bound == OZGEMM_BOUND_FAST && q >= OZGEMM_FAST_Q_LIMIT) return OZGEMM_RANGE;  // 64-bit norm sums
  if (g.bound == OZGEMM_BOUND_ACCU) {
    int st = check_method_range(q, s);
    if (st) return st;
    if (!accu_fits(g.lay, m, n, q)) return OZGEMM_WORKSPACE_TOO_SMALL;
  }
  return run_scale(config_ctx(), m, n, q, s, A, lda, B, ldb, e, f);
}

int ozgemm_set_bound(int mode) {
  if (mode != OZGEMM_BOUND_CONSERVATIVE && mode != OZGEMM_BOUND_FAST && mode != OZGEMM_BOUND_ACCU) return -1;
  g.bound = mode;
  return OZGEMM_OK;
}

int ozgemm_bound_budget(int s, int q, int mode, int* kappa_a, int* kappa_b) {
  if (s < 1 || s > OZGEMM_S_MAX) return -1;
  if (q < 1 || q > OZGEMM_Q_MAX) return -2;
  if (mode != OZGEMM_BOUND_CONSERVATIVE && mode != OZGEMM_BOUND_FAST && mode != OZGEMM_BOUND_ACCU) return -3;
  if (kappa_a == nullptr) return -4;
  if (kappa_b == nullptr) return -5;
  if (mode == OZGEMM_BOUND_ACCU) {
    if (q > OZGEMM_ACCU_Q_MAX || s < 2 || kbits_exact(s, q) < 1) return OZGEMM_RANGE;
    int ka, kb;
    fast_budget(s, &ka, &kb);
    *kappa_a = ka + kb;  // the budget a_i + b_j + L_ij <= K2 shares
    *kappa_b = ACCU_KMAX;
  } else if (mode == OZGEMM_BOUND_FAST) {
    if (q >= OZGEMM_FAST_Q_LIMIT) return OZGEMM_RANGE;  // 64-bit norm sums
    fast_budget(s, kappa_a, kappa_b);
  } else {
    const int k = kbits_exact(s, q);
    if (k < 1) return OZGEMM_RANGE;
    *kappa_a = *kappa_b = k;
  }
  return OZGEMM_OK;
}

int ozgemm_stage_residue(int m, int n, int q, int s, const double* A, int lda, const double* B, int ldb,
                         const int32_t* e, const int32_t* f, int8_t* Ares, int8_t* Bres, double* Aprime,
                         double* Bprime) {
  if (m < 0) return -1;
  if (n < 0) return -2;
  if (q < 1) return -3;
  if (s < 1 || s > OZGEMM_S_MAX) return -4;
  if (A == nullptr && m > 0) return -5;
  if (lda < std::max(1, m)) return -6;
  if (B == nullptr && n > 0) return -7;
  if (ldb < std::max(1, q)) return -8;
  if (e == nullptr) return -9;
  if (f == nullptr) return -10;
  if (Ares == nullptr) return -11;
  if (Bres == nullptr) return -12;
  int st = check_range(m, n, q, s);
  if (st) return st;
  return run_residue(m, n, q, s, A, lda, B, ldb, e, f, Ares, Bres, Aprime, Bprime);
}

int ozgemm_stage_gemm(int m, int n, int q, int s, const int8_t* Ares, const int8_t* Bres, int32_t* Ct,
                      uint8_t* rt) {
  if (m < 0) return -1;
  if (n < 0) return -2;
  if (q < 1) return -3;
  if (s < 1 || s > OZGEMM_S_MAX) return -4;
  if (Ares == nullptr) return -5;
  if (Bres == nullptr) return -6;
  int st = check_range(m, n, q, s);
  if (st) return st;
  if (Ct != nullptr && q >= OZGEMM_Q_LIMIT) return OZGEMM_RANGE;  // int32 C_t would overflow
  int mp, np, qp;
  dims(m, n, q, &mp, &np, &qp);
  ResidueConsts rc;
  GemmConsts gc;
  CrtConsts cc;
  make_consts(s, q, g.bound, &rc, &gc, &cc);
  SplitChoice split{1, qp / K_PAD};
  int cus = 0;
  if (Ct == nullptr && rt != nullptr && (st = product_split(g.lay, mp, np, qp, s, &split, &cus))) return st;
  uint8_t* parts = reinterpret_cast<uint8_t*>(g.ws + g.lay.rt);
  OZ_CHECK(launch_gemm(Ares, Bres, mp, np, qp, gc, Ct, rt, split, parts, cus, g.stream));
  return 0;
}

int ozgemm_gemm_parts(int m, int n, int q, int s, int* parts) {
  if (m < 1) return -1;
  if (n < 1) return -2;
  if (q < 1) return -3;
  if (s < 1 || s > OZGEMM_S_MAX) return -4;
  if (parts == nullptr) return -5;
  if (!g.configured) return OZGEMM_NOT_CONFIGURED;
  if (m > g.max_m || n > g.max_n || q > g.max_q || s > g.s_max) return OZGEMM_RANGE;
  int mp, np, qp;
  dims(m, n, q, &mp, &np, &qp);
  SplitChoice split{};
  int cus = 0;
  const int st = product_split(g.lay, mp, np, qp, s, &split, &cus);
  if (st) return st;
  *parts = split.parts;
  return OZGEMM_OK;
}

int ozgemm_stage_crt(int m, int n, int q, int s, const uint8_t* rt, const int32_t* e, const int32_t* f, double* C,
                     int ldc) {
  if (m < 0) return -1;
  if (n < 0) return -2;
  if (q < 1) return -3;
  if (s < 1 || s > OZGEMM_S_MAX) return -4;
  if (rt == nullptr) return -5;
  if (e == nullptr) return -6;
  if (f == nullptr) return -7;
  if (C == nullptr && m > 0 && n > 0) return -8;
  if (ldc < std::max(1, m)) return -9;
  int st = check_range(m, n, q, s);
  if (st) return st;
  if (m == 0 || n == 0) return 0;
  int mp, np, qp;
  dims(m, n, q, &mp, &np, &qp);
  ResidueConsts rc;
  GemmConsts gc;
  CrtConsts cc;
  make_consts(s, q, g.bound, &rc, &gc, &cc);
  if ((st = ensure_crt_table())) return st;
  cc.wtab = crt_table(s);
  OZ_CHECK(launch_crt(rt, m, n, mp, np, e, f, cc, C, ldc, g.stream));
  return 0;
}

int ozgemm_scheme1_beta(int q) { return s1_beta(q); }

int ozgemm_scheme1_outputs(int k, int variant, int q) {
  int st = s1_check(k, variant, q);
  if (st) return st < 0 ? st : -3;
  const int beta = s1_beta(std::max(q, 1));
  return s1_nout(k, variant, s1_group(std::max(q, 1), beta));
}

size_t ozgemm_scheme1_workspace_bytes(int m, int n, int q, int k, int variant) {
  if (m < 0 || n < 0 || q < 0 || s1_check(k, variant, q) != 0) return 0;
  return s1_base() + s1_layout(m, n, q, k, variant).total;
}

int ozgemm_scheme1_dgemm(int m, int n, int q, const double* A, int lda, const double* B, int ldb, double* C,
                         int ldc, int k, int variant) {
  int st = check_common(m, n, q, A, lda, B, ldb);
  if (st) return st;
  if (C == nullptr && m > 0 && n > 0) return -8;
  if (ldc < std::max(1, m)) return -9;
  if (k < 1 || k > OZGEMM_S1_K_MAX) return -10;
  if (variant != OZGEMM_S1_RN && variant != OZGEMM_S1_HYBRID) return -11;
  if (!g.configured) return OZGEMM_NOT_CONFIGURED;
  if (m > OZ_MAX_ROWS || n > OZ_MAX_ROWS || (q > 0 && s1_beta(q) < 1)) return OZGEMM_RANGE;
  if (m == 0 || n == 0) return OZGEMM_OK;
  const size_t cb = mat_bytes(m, n, ldc);
  if (overlaps(C, cb, A, mat_bytes(m, q, lda)) || overlaps(C, cb, B, mat_bytes(q, n, ldb))) return -8;
  if (q == 0) {
    OZ_CHECK(launch_fill_zero(C, m, n, ldc, g.stream));
    return OZGEMM_OK;
  }
  const S1Layout L = s1_layout(m, n, q, k, variant);
  if (g.ws_bytes < s1_base() + L.total) return OZGEMM_WORKSPACE_TOO_SMALL;
  char* base = g.ws + s1_base();
  int4* gemm_plan = reinterpret_cast<int4*>(base + L.plans);
  int4* acc_plan = gemm_plan + OZGEMM_S1_MAX_OUT;
  int32_t* gA = reinterpret_cast<int32_t*>(base + L.gA);
  int32_t* gB = reinterpret_cast<int32_t*>(base + L.gB);
  uint64_t* pmax = reinterpret_cast<uint64_t*>(base + L.pmax);
  int8_t* Asl = reinterpret_cast<int8_t*>(base + L.asl);
  int8_t* Bsl = reinterpret_cast<int8_t*>(base + L.bsl);
  int32_t* P = reinterpret_cast<int32_t*>(base + L.P);
  // Scheme II keeps its constant table below this region; it stays valid.

  std::array<hipEvent_t, 5> ev{};
  const bool timed = g.timing && g.events.size() < TIMING_MAX_CALLS;
  if (timed) {
    for (auto& x : ev) OZ_CHECK(hipEventCreateWithFlags(&x, kTimingEventFlags));
    OZ_CHECK(hipEventRecord(ev[0], g.stream));
    OZ_CHECK(hipEventRecord(ev[1], g.stream));
  }
  if ((st = s1_split(L, m, n, q, k, variant, A, lda, B, ldb, Asl, Bsl, gA, gB, pmax))) return st;
  if (timed) OZ_CHECK(hipEventRecord(ev[2], g.stream));
  OZ_CHECK(launch_s1_plan(variant, k, L.r, L.beta, gemm_plan, acc_plan, g.stream));
  OZ_CHECK(launch_gemm_multi(Asl, Bsl, L.mp, L.np, L.qp, gemm_plan, L.nout, P, g.stream));
  if (timed) OZ_CHECK(hipEventRecord(ev[3], g.stream));
  OZ_CHECK(launch_s1_accum(P, m, n, L.mp, L.np, L.nout, acc_plan, gA, L.mp, gB, L.np, C, ldc, g.stream));
  if (timed) {
    OZ_CHECK(hipEventRecord(ev[4], g.stream));
    g.events.push_back(ev);
  }
  return OZGEMM_OK;
}

int ozgemm_scheme1_stage_split(int m, int n, int q, int k, int variant, const double* A, int lda, const double* B,
                               int ldb, int8_t* Aslices, int8_t* Bslices, int32_t* gA, int32_t* gB) {
  int st = check_common(m, n, q, A, lda, B, ldb);
  if (st) return st;
  if (q < 1) return -3;
  if (k < 1 || k > OZGEMM_S1_K_MAX) return -8;
  if (variant != OZGEMM_S1_RN && variant != OZGEMM_S1_HYBRID) return -9;
  if (Aslices == nullptr) return -10;
  if (Bslices == nullptr) return -11;
  if (gA == nullptr) return -12;
  if (gB == nullptr) return -13;
  if (!g.configured) return OZGEMM_NOT_CONFIGURED;
  if (m > OZ_MAX_ROWS || n > OZ_MAX_ROWS || s1_beta(q) < 1) return OZGEMM_RANGE;
  const S1Layout L = s1_layout(m, n, q, k, variant);
  if (g.ws_bytes < s1_base() + L.pmax + (size_t)L.nch * std::max(L.mp, L.np) * 8) return OZGEMM_WORKSPACE_TOO_SMALL;
  uint64_t* pmax = reinterpret_cast<uint64_t*>(g.ws + s1_base() + L.pmax);
  return s1_split(L, m, n, q, k, variant, A, lda, B, ldb, Aslices, Bslices, gA, gB, pmax);
}

int ozgemm_scheme1_stage_products(int m, int n, int q, int k, int variant, const int8_t* Aslices,
                                  const int8_t* Bslices, int32_t* P) {
  if (m < 0) return -1;
  if (n < 0) return -2;
  if (q < 1) return -3;
  if (k < 1 || k > OZGEMM_S1_K_MAX) return -4;
  if (variant != OZGEMM_S1_RN && variant != OZGEMM_S1_HYBRID) return -5;
  if (Aslices == nullptr) return -6;
  if (Bslices == nullptr) return -7;
  if (P == nullptr) return -8;
  if (!g.configured) return OZGEMM_NOT_CONFIGURED;
  if (m > OZ_MAX_ROWS || n > OZ_MAX_ROWS || s1_beta(q) < 1) return OZGEMM_RANGE;
  const S1Layout L = s1_layout(m, n, q, k, variant);
  if (g.ws_bytes < s1_base() + L.plans + 2 * OZGEMM_S1_MAX_OUT * sizeof(int4)) return OZGEMM_WORKSPACE_TOO_SMALL;
  int4* gemm_plan = reinterpret_cast<int4*>(g.ws + s1_base() + L.plans);
  OZ_CHECK(launch_s1_plan(variant, k, L.r, L.beta, gemm_plan, gemm_plan + OZGEMM_S1_MAX_OUT, g.stream));
  OZ_CHECK(launch_gemm_multi(Aslices, Bslices, L.mp, L.np, L.qp, gemm_plan, L.nout, P, g.stream));
  return 0;
}

int ozgemm_scheme1_stage_accumulate(int m, int n, int q, int k, int variant, const int32_t* P, const int32_t* gA,
                                    const int32_t* gB, double* C, int ldc) {
  if (m < 0) return -1;
  if (n < 0) return -2;
  if (q < 1) return -3;
  if (k < 1 || k > OZGEMM_S1_K_MAX) return -4;
  if (variant != OZGEMM_S1_RN && variant != OZGEMM_S1_HYBRID) return -5;
  if (P == nullptr) return -6;
  if (gA == nullptr) return -7;
  if (gB == nullptr) return -8;
  if (C == nullptr && m > 0 && n > 0) return -9;
  if (ldc < std::max(1, m)) return -10;
  if (!g.configured) return OZGEMM_NOT_CONFIGURED;
  if (m > OZ_MAX_ROWS || n > OZ_MAX_ROWS || s1_beta(q) < 1) return OZGEMM_RANGE;
  if (m == 0 || n == 0) return 0;
  const S1Layout L = s1_layout(m, n, q, k, variant);
  if (g.ws_bytes < s1_base() + L.plans + 2 * OZGEMM_S1_MAX_OUT * sizeof(int4)) return OZGEMM_WORKSPACE_TOO_SMALL;
  int4* gemm_plan = reinterpret_cast<int4*>(g.ws + s1_base() + L.plans);
  int4* acc_plan = gemm_plan + OZGEMM_S1_MAX_OUT;
  OZ_CHECK(launch_s1_plan(variant, k, L.r, L.beta, gemm_plan, acc_plan, g.stream));
  OZ_CHECK(launch_s1_accum(P, m, n, L.mp, L.np, L.nout, acc_plan, gA, L.mp, gB, L.np, C, ldc, g.stream));
  return 0;
}

int ozgemm_timing(int enable) {
  for (auto& ev : g.events)
    for (auto& x : ev) (void)hipEventDestroy(x);
  g.events.clear();
  g.timing = enable != 0;
  return OZGEMM_OK;
}

int ozgemm_phase_ms(double* ms_out, int* calls) {
  if (ms_out == nullptr) return -1;
  for (int p = 0; p < 4; ++p) ms_out[p] = 0.0;
  for (auto& ev : g.events) {
    OZ_CHECK(hipEventSynchronize(ev[4]));
    for (int p = 0; p < 4; ++p) {
      float ms = 0.f;
      OZ_CHECK(hipEventElapsedTime(&ms, ev[p], ev[p + 1]));
      ms_out[p] += ms;
    }
  }
  if (calls) *calls = (int)g.events.size();
  return OZGEMM_OK;
}

int ozgemm_phase_calls(double* ms_out, int max_calls, int* calls) {
  if (max_calls < 0) return -2;
  if (ms_out == nullptr && max_calls > 0) return -1;
  const int n = std::min(max_calls, (int)g.events.size());
  for (int c = 0; c < n; ++c) {
    const auto& ev = g.events[(size_t)c];
    OZ_CHECK(hipEventSynchronize(ev[4]));
    for (int p = 0; p < 4; ++p) {
      float ms = 0.f;
      OZ_CHECK(hipEventElapsedTime(&ms, ev[p], ev[p + 1]));
      ms_out[4 * c + p] = ms;
    }
  }
  if (calls) *calls = (int)g.events.size();
  return OZGEMM_OK;
}

int ozgemm_mfma_ceiling(int blocks, int steps, unsigned seed, unsigned* sink, void* hip_stream) {
  if (blocks < 1 || blocks > (1 << 20)) return -1;
  if (steps < 1) return -2;
  if (sink == nullptr) return -4;
  OZ_CHECK(launch_mfma_ceiling(blocks, steps, seed, sink, (hipStream_t)hip_stream));
  return OZGEMM_OK;
}

}  // extern "C"
