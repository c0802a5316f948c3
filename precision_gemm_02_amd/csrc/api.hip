// C ABI of pgemm: argument checks, quick returns, variant choice and launch.
// Declarations and the full contract are in include/pgemm.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <cstring>
#include <mutex>

#include "pgemm.h"
#include "variants.hpp"

namespace pgemm {
namespace {

// Largest grid the launcher accepts (workgroups); far beyond any problem
// that fits in device memory.
constexpr long long kMaxTiles = 1LL << 24;

template <typename T>
bool aligned16(const T* p) {
  return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

template <typename T>
bool elem_aligned(const T* p) {
  return (reinterpret_cast<uintptr_t>(p) % sizeof(T)) == 0;
}

// Returns 0 or -(1-based position of the first bad argument) in the
// gemm_f32 / gemm_f64 signature.
template <typename T>
int check_args(int m, int n, int k, T alpha, const T* A, int lda, const T* B, int ldb,
               const T* C, int ldc) {
  if (m < 0) return -1;
  if (n < 0) return -2;
  if (k < 0) return -3;
  const bool touch_c = m > 0 && n > 0;
  const bool read_ab = touch_c && k > 0 && alpha != T(0);
  if (read_ab && (A == nullptr || !elem_aligned(A))) return -5;
  if (lda < (m > 1 ? m : 1)) return -6;
  if (read_ab && (B == nullptr || !elem_aligned(B))) return -7;
  if (ldb < (k > 1 ? k : 1)) return -8;
  if (touch_c && (C == nullptr || !elem_aligned(C))) return -10;
  if (ldc < (m > 1 ? m : 1)) return -11;
  return 0;
}

// 128-bit path: every row of every operand starts on a 16-byte boundary.
template <typename T>
bool vec_ok(const T* A, int lda, const T* B, int ldb, const T* C, int ldc) {
  constexpr int V = 16 / sizeof(T);
  return aligned16(A) && aligned16(B) && aligned16(C) && lda % V == 0 && ldb % V == 0 &&
         ldc % V == 0;
}

long long ceil_div(long long a, long long b) { return (a + b - 1) / b; }

// Index of the named variant; the first entry if the name is not compiled in
// (the host tests check that every name the choice uses exists).
template <typename T>
int find_variant(const Variant<T>* table, int count, const char* name) {
  for (int i = 0; i < count; ++i)
    if (std::strcmp(table[i].name, name) == 0) return i;
  return 0;
}

// One tile class: the aligned and unaligned variants of one tiling, the
// share of the matrix-core peak its steady state reaches, and any fixed cost
// per round beyond the common one (seconds).  First measured with one round
// of 256 tiles timed against K (256x256 154.4, 128x128 153.4, 256x128 152.6
// TFLOP/s of 157.3; fp64 128x128 76.9 of 78.6); the 256x128 and 128x128
// classes and the fp64 64x64 class were then refitted to every class timed
// on 70 random shapes and 66 small-tile shapes, which cut the mean loss of
// the choice against the fastest class from 1.4 % to 1.1 %.
struct TileClass {
  int vec, ua;
  double eff;
  double extra_s;
  // > 0: this many workgroups share a compute unit and run together; up to
  // that many tiles per compute unit cost one fixed part and their K loops
  // (see estimate).
  int coresident = 0;
  // Such a class's efficiency with one tile per compute unit and a long K
  // loop: one wave per SIMD then waits for operands that come from beyond
  // the L2 (panels that few tiles share, or columns that straddle cache
  // lines).
  double eff_lone = 0;
};

// Variant tables plus the tile classes the shape/alignment choice uses,
// looked up by name once.
struct Tables {
  const Variant<float>* f32;
  const Variant<double>* f64;
  int n32, n64;
  TileClass f32c[6];
  TileClass f64c[2];
  Tables() {
    f32 = f32_variants(&n32);
    f64 = f64_variants(&n64);
    f32c[0] = {find_variant(f32, n32, "f32_256x256x16_w2x4_s3_vec"),
               find_variant(f32, n32, "f32_256x256x16_w2x4_s3_ua"), 0.982, 0};
    f32c[1] = {find_variant(f32, n32, "f32_256x128x32_w4x2_s3_vec"),
               find_variant(f32, n32, "f32_256x128x32_w4x2_s3_ua"), 0.980, 2.0e-6};
    // 128 x 128: a ring of 4 stages of BK 16 and 8 waves of 32 x 64; it has
    // the least fixed cost per tile of the 128 x 128 configurations (no
    // hand-over between K groups), which is what decides at these sizes
    // (2048^3 144.5 against 143.2 TFLOP/s for two K groups of 4 waves).
    f32c[2] = {find_variant(f32, n32, "f32_128x128x16_w4x2_s4_vec"),
               find_variant(f32, n32, "f32_128x128x16_w4x2_s4_ua"), 0.985, 0.75e-6};
    // 64 x 64: small problems, and mid-sized ones whose 128 x 128 tiles
    // would leave a badly filled last round (2500^3 to 3500^3, the ragged
    // 4097 x 3001 x 1023).  Several of these workgroups share a compute unit
    // (32 KiB of LDS, ~50 VGPRs); fitted to the measured times of 1280^3 to
    // 4096^3 under the round model, the class runs at ~0.88 of peak.  1024^3
    // as one round of 256 tiles: 18.9 us (113.8 TFLOP/s) against 32.8 us for
    // 64 tiles of 128 x 128, each with its K loop split over 4 workgroups.
    f32c[3] = {find_variant(f32, n32, "f32_64x64x16_w2x2_s4_vec"),
               find_variant(f32, n32, "f32_64x64x16_w2x2_s4_ua"), 0.88, 0};
    // 64 x 64 with two K groups of 4 waves (two waves per SIMD): its steady
    // state keeps ~0.96 of peak where the one-wave-per-SIMD class above
    // falls to ~0.64 (operands no longer served from the caches: 1024^2 x
    // 2048 and beyond), and it pays ~1.9 us more per round for the hand-over
    // of partial sums between the groups.  Fitted to 11 M x N shapes from
    // 256 x 4096 to 2560^2 at K = 256 ... 8192: the model then picks it from
    // K ~ 1500 on (measured gains up to 50 % at K >= 2048; at K <= 1024 the
    // one-group class is up to 12 % faster).
    f32c[4] = {find_variant(f32, n32, "f32_64x64x32_w2x2_s3_k2_vec"),
               find_variant(f32, n32, "f32_64x64x32_w2x2_s3_k2_ua"), 0.96, 1.9e-6};
    // 32 x 32 tiles in four K groups of one wave (one per SIMD), which hand
    // their partial sums over through LDS: problems too small to give every
    // compute unit a 64 x 64 tile, and up to three tiles per compute unit
    // (48 KiB of LDS each), which run together.  Fitted to 23 shapes from
    // 128^3 to 1536 x 512 x 256 (K up to 4096): ~0.80 of peak in the K loop
    // of one tile, ~3.5 us fixed in all; 640^3 8.7 us against 11.9 for
    // 64 x 64 tiles, 1024 x 512 x 1024 11.7 against 17.3, but 1024^3 24.0
    // against 17.8 (four tiles per compute unit: their operand traffic then
    // bounds them).  Beyond three tiles per unit it is priced in groups of
    // three per unit (see estimate: up to three groups, with K loops of 12 K
    // tiles or more; otherwise by rounds).  A lone
    // tile per unit with a long K loop (8 K tiles or more) runs at 0.5 to
    // 0.8: 768 x 64 x 2836 22.9 us (panels shared by 2 tiles), 252^2 x 4096
    // 27.9 (columns of 1008 bytes), 256^2 x 4096 20.1.  It is priced at 0.5,
    // so that stream-K with 64 x 64 tiles, where a workspace allows it, wins
    // there (7 of 9 such shapes measured faster with it).
    f32c[5] = {find_variant(f32, n32, "f32_32x32x64_w1x1_s3_k4_vec"),
               find_variant(f32, n32, "f32_32x32x64_w1x1_s3_k4_ua"), 0.80, 1.75e-6, 3, 0.5};
    // fp64: 128 x 128 tiles for large problems.  Their 64 x 32 wave tiles
    // leave registers for the unrolled steady-state loop, which more than
    // pays for the extra operand traffic of smaller tiles (4096^3: 74.0
    // TFLOP/s against 72.3 for 256 x 128 tiles, whose loop cannot be
    // unrolled).  64 x 64 tiles (8 waves of 32 x 16, a ring of 4) elsewhere:
    // 1024^3 60.5 against 17.6 TFLOP/s, 3000^3 70.5 against 53.3; under the
    // round model ~0.93 of peak (0.87 to 0.99 on the shapes measured).  The
    // 128 x 128 class's rounds cost ~3 us more than the common fixed part
    // (fitted with the 64 x 64 one to 40 random fp64 shapes, where short K
    // loops had picked 128 x 128 tiles up to 13 % too slow).
    f64c[0] = {find_variant(f64, n64, "f64_128x128x16_w2x4_s3_vec"),
               find_variant(f64, n64, "f64_128x128x16_w2x4_s3_ua"), 0.978, 3e-6};
    f64c[1] = {find_variant(f64, n64, "f64_64x64x16_w2x4_s4_vec"),
               find_variant(f64, n64, "f64_64x64x16_w2x4_s4_ua"), 0.93, 0};
  }
};

const Tables& tables() {
  static const Tables t;
  return t;
}

// Compute units of the current device (cached per device; 256 if unknown).
// Threads may race to fill an entry; they all store the same value.
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v <= 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        v <= 0)
      v = 256;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

// Stream-K for the last round of tiles.  With T tiles on P compute units,
// the first R = floor(T/P) rounds stay one tile per workgroup; the K tiles of
// the remaining Tr = T - R*P tiles (I = Tr*nk iterations, in (tile, K tile)
// order) are shared by S more workgroups, workgroup w taking iterations
// [floor(w*I/S), floor((w+1)*I/S)).  S > Tr, so a range is shorter than a
// tile and covers the end of one tile and the start of the next at most;
// each piece's partial sums go to the workspace (two slots per workgroup)
// and the fix-up kernel adds each tile's pieces in K order.  Every range
// keeps at least 4 K tiles after a full round (the shared tiles then run
// beside nothing else) or 2 without one (small problems).  Two values of S
// are weighed: as many workgroups as that allows, up to P, or a multiple of
// Tr (s workgroups per tile, up to P), whose ranges never cross a tile, so
// each workgroup runs one piece.
struct SkPlan {
  int full_tiles = 0, wgs = 0;
  size_t bytes = 0;
};

// Whether some range of S workgroups over I = tr*nk iterations crosses a
// tile boundary (then some workgroups run two pieces).  Boundary j*nk starts
// a range iff some w has j*S/tr <= w < j*S/tr + S/I: with x = j*S mod tr,
// iff x == 0 or (tr - x)*nk < S.
inline bool sk_crosses(long long tr, long long nk, long long S) {
  if (S % tr == 0) return false;
  for (long long j = 1; j < tr; ++j) {
    const long long x = (j * S) % tr;
    if (x != 0 && (tr - x) * nk >= S) return true;
  }
  return false;
}

// Estimated time of the last round under stream-K with S workgroups (same
// units and fixed part as estimate below): the longest range's share of a
// tile's K loop, the fixed part of one or two pieces, and the fix-up kernel
// (its HBM traffic at ~4 TB/s and ~8 us for its launch behind the GEMM
// kernel and the uneven end of the pieces, fitted to 29 measured shapes).
template <typename T>
double sk_time(const Variant<T>& v, double kloop, double fixed, long long tr, long long nk,
               long long S, double unit_s) {
  const long long per_wg = ceil_div(tr * nk, S);
  const double tile_bytes = (double)v.bm * v.bn * sizeof(T);
  const double fix_bytes = ((double)S + 3.0 * (double)tr) * tile_bytes;
  return kloop * (double)per_wg / (double)nk + (sk_crosses(tr, nk, S) ? 2 : 1) * fixed +
         (fix_bytes / 4e12 + 8e-6) / unit_s;
}

// Per-precision constants of the time model: one multiply-add on one compute
// unit at the precision's matrix peak, in seconds.
template <typename T>
constexpr double unit_seconds() {
  return 2.0 / ((sizeof(T) == 4 ? 157.3e12 : 78.6e12) / 256);
}

// A tile's K loop at the class's efficiency, and the fixed part of a round:
// ~1.5 us of prologue, the round's stores of C at ~5 TB/s and the class's
// own extra (all in units).
template <typename T>
void round_costs(const Variant<T>& v, const TileClass& tc, int k, int cus, double* kloop,
                 double* fixed) {
  const double c_bytes = (double)cus * v.bm * v.bn * sizeof(T);
  *kloop = (double)v.bm * (double)v.bn * (double)k / tc.eff;
  *fixed = (1.5e-6 + tc.extra_s + c_bytes / 5e12) / unit_seconds<T>();
}

template <typename T>
SkPlan sk_plan(const Variant<T>& v, const TileClass& tc, int m, int n, int k, int cus) {
  SkPlan p;
  const long long tiles = ceil_div(m, v.bm) * ceil_div(n, v.bn);
  const long long rounds = tiles / cus, rest = tiles - rounds * cus;
  const long long nk = ceil_div(k, v.bk);
  if (rest == 0) return p;
  const long long min_iters = rounds >= 1 ? 4 : 2;
  long long s_all = rest * nk / min_iters;
  if (s_all > cus) s_all = cus;
  long long per_tile = cus / rest;
  if (per_tile > nk / min_iters) per_tile = nk / min_iters;
  const long long s_al = rest * per_tile;
  double kloop, fixed;
  round_costs(v, tc, k, cus, &kloop, &fixed);
  long long S = 0;
  double best = 0;
  for (const long long c : {s_al, s_all}) {
    if (c <= rest) continue;
    const double t = sk_time(v, kloop, fixed, rest, nk, c, unit_seconds<T>());
    if (S == 0 || t < best) {
      S = c;
      best = t;
    }
  }
  if (S == 0) return p;
  p.full_tiles = (int)(rounds * cus);
  p.wgs = (int)S;
  p.bytes = (size_t)2 * (size_t)S * (size_t)v.bm * (size_t)v.bn * sizeof(T);
  return p;
}

// Estimated time of variant v on an m x n x k problem, in multiply-adds of
// one compute unit at the precision's full matrix rate.  Each round of tiles
// (every compute unit busy with one tile) costs the tile's K loop at the
// class's efficiency plus the fixed part (round_costs).  The last, partly
// filled round costs a whole round, or with a stream-K plan (`sk`) its
// sk_time.  Edge tiles cost as much as inner ones (they run the same loop).
// A class whose workgroups share a compute unit and run together
// (TileClass::coresident) costs, up to that many tiles per unit, one fixed
// part plus its tiles' K loops (at eff_lone for a lone tile with a long K
// loop).
// Against every class timed on 70 random shapes not used in the fit, the
// choice runs on average within 1.1 % of the fastest one (7 shapes lose more
// than 3 %, at most 10 %).
template <typename T>
double estimate(const Variant<T>& v, const TileClass& tc, int m, int n, int k, int cus,
                const SkPlan* sk) {
  const long long tiles = ceil_div(m, v.bm) * ceil_div(n, v.bn);
  const long long rounds = tiles / cus, rest = tiles - rounds * cus;
  double kloop, fixed;
  round_costs(v, tc, k, cus, &kloop, &fixed);
  const long long per_cu = ceil_div(tiles, (long long)cus);
  if (tc.coresident > 0 && per_cu <= tc.coresident) {
    const bool lone = per_cu == 1 && k >= 8 * v.bk;
    return fixed + kloop * (double)per_cu * (lone ? tc.eff / tc.eff_lone : 1.0);
  }
  if (tc.coresident > 0 && per_cu <= 3 * tc.coresident && k >= 12 * v.bk &&
      (sk == nullptr || sk->wgs == 0)) {
    // more tiles than run together, up to three groups, K loops of 12 K
    // tiles or more: groups of `coresident` tiles per unit, each one fixed
    // part plus their K loops, the last group partly filled (measured on 18
    // shapes whose choice this changes: 2 to 22 % faster on 15; at ~20 tiles
    // per unit the small tiles' memory traffic made them 8 % slower, and
    // with 8 K tiles their fixed costs 9 %)
    const long long group = (long long)cus * tc.coresident;
    const long long full = tiles / group, rest_g = tiles - full * group;
    double t = (double)full * (fixed + kloop * (double)tc.coresident);
    if (rest_g > 0) {
      const long long last = ceil_div(rest_g, (long long)cus);
      const bool lone = last == 1 && k >= 8 * v.bk;
      t += fixed + kloop * (double)last * (lone ? tc.eff / tc.eff_lone : 1.0);
    }
    return t;
  }
  const double t = (double)rounds * (kloop + fixed);
  if (rest == 0) return t;
  if (sk != nullptr && sk->wgs > 0)
    return t + sk_time(v, kloop, fixed, rest, ceil_div(k, v.bk), sk->wgs, unit_seconds<T>());
  return t + kloop + fixed;
}

// Rows left below the last whole tile row that a separate strip kernel can
// take (0: none): at most kStripRows of them, and at least one whole tile
// row above.
template <typename T>
int strip_rows(const Variant<T>& v, int m) {
  const int r = m % v.bm;
  return (r > 0 && r <= kStripRows && m > v.bm) ? r : 0;
}

// Estimated time of the strip of r rows (same units as estimate): the
// largest of its latency chain (~2.5 us per batch of four steps of every
// thread, ~2 us for the sums), reading B once from HBM (~4 TB/s), every
// workgroup's reads of the strip of A from the caches (one 128-byte line per
// inner index, ~7 TB/s; `wg_cols` columns per workgroup) and its
// multiply-adds on the vector units (~40 TFLOP/s fp32, ~20 fp64), plus ~4 us
// for a launch behind the GEMM kernel when it is a kernel of its own.  Run
// by extra workgroups of the GEMM's own grid (Variant::fstrip) it has no
// launch, and it runs beside the last round of tiles, but its loads compete
// with theirs: on 24 shapes and every class the measured cost (time with the
// strip minus time of the tiles alone) was 0.2 to 2.8 times the largest term,
// mostly 1 to 2.  Doubling the estimate changed the choice on 41 of 6000
// random shapes and lost 1.7 % on them (geometric mean; up to 26 % where a
// short strip was then avoided, against at most 5.5 % gained), so it is not
// doubled.
template <typename T>
double strip_time(int r, int n, int k, int wg_cols, bool fused) {
  const double s = sizeof(T);
  const double lat = 2.5e-6 * (double)ceil_div(k, 4 * kStripThreads) + 2e-6;
  const double b_s = (double)k * n * s / 4e12;
  const double a_s = (double)ceil_div(n, wg_cols) * (double)k * 128.0 / 7e12;
  const double f_s = 2.0 * r * (double)n * k / (sizeof(T) == 4 ? 40e12 : 20e12);
  double t = lat;
  if (b_s > t) t = b_s;
  if (a_s > t) t = a_s;
  if (f_s > t) t = f_s;
  return ((fused ? 0.0 : 4e-6) + t) / unit_seconds<T>();
}

// What a call launches: the tile class, its stream-K plan (wgs == 0: none)
// and the rows left to the strip kernel (0: none).
struct Choice {
  int cls = 0;
  SkPlan plan;
  int strip = 0;
};

// The tile class with the least estimated time for this shape, each class
// weighed with and without the strip kernel for the rows below its last
// whole tile row (the strip only where it is estimated at least 2 % faster
// than the class without it), and with stream-K of the last round where
// sk_ok (only where that is estimated at least 1 % faster: below that the
// measured gains were within noise or losses).
template <typename T>
Choice choose(int m, int n, int k, bool sk_ok, long long ldc) {
  const Tables& t = tables();
  const Variant<T>* table;
  const TileClass* cls;
  int ncls;
  if constexpr (sizeof(T) == 4) {
    table = t.f32;
    cls = t.f32c;
    ncls = 6;
  } else {
    table = t.f64;
    cls = t.f64c;
    ncls = 2;
  }
  const int cus = device_cus();
  if (k <= 0) k = 1;
  Choice best;
  double best_t = -1;
  for (int c = 0; c < ncls; ++c) {
    const Variant<T>& v = table[cls[c].vec];
    if (v.max_ldc > 0 && ldc > v.max_ldc) continue;   // C's offsets would not fit
    const int r = strip_rows(v, m);
    double e_cls = 0;
    for (int o = 0; o < (r > 0 ? 2 : 1); ++o) {
      const int strip = o == 0 ? 0 : r;       // rows left to the strip kernel
      const int mm = m - strip;
      double e = estimate(v, cls[c], mm, n, k, cus, nullptr);
      SkPlan plan;
      const SkPlan p = (sk_ok && v.sk) ? sk_plan(v, cls[c], mm, n, k, cus) : SkPlan{};
      if (p.wgs > 0) {
        const double e_sk = estimate(v, cls[c], mm, n, k, cus, &p);
        if (e_sk * 1.01 < e) {
          e = e_sk;
          plan = p;
        }
      }
      if (strip > 0) {
        int sc, cgw;
        v.strip_shape(strip, n, cus, &sc, &cgw);
        e += strip_time<T>(strip, n, k, sc * cgw, v.fstrip);
        if (e * 1.02 >= e_cls) continue;
      }
      e_cls = e;
      if (best_t < 0 || e < best_t) {
        best.cls = c;
        best.plan = plan;
        best.strip = strip;
        best_t = e;
      }
    }
  }
  return best;
}

// The variant a call launches, its stream-K plan and its strip rows: with a
// workspace large enough for the plan of the choice that is best with
// stream-K, that choice; otherwise the best one without stream-K.
template <typename T>
int pick(int m, int n, int k, int ldc, bool vec, size_t ws_bytes, SkPlan* plan, int* strip) {
  const Tables& t = tables();
  const TileClass* cls;
  if constexpr (sizeof(T) == 4) cls = t.f32c;
  else cls = t.f64c;
  if (ws_bytes > 0) {
    const Choice c = choose<T>(m, n, k, true, ldc);
    if (c.plan.wgs == 0 || ws_bytes >= c.plan.bytes) {
      *plan = c.plan;
      *strip = c.strip;
      return vec ? cls[c.cls].vec : cls[c.cls].ua;
    }
  }
  const Choice c = choose<T>(m, n, k, false, ldc);
  *plan = SkPlan{};
  *strip = c.strip;
  return vec ? cls[c.cls].vec : cls[c.cls].ua;
}

template <typename T>
hipError_t launch_scale(int m, int n, T beta, T* C, int ldc, hipStream_t s) {
  if (beta == T(1)) return hipSuccess;
  void* args[] = {&m, &n, &beta, &C, &ldc};
  const dim3 grid((unsigned)ceil_div(m, 256), (unsigned)(n < 65535 ? n : 65535));
  return hipLaunchKernel(reinterpret_cast<const void*>(&scale_kernel<T>), grid, dim3(256),
                         args, 0, s);
}

// Launch variant v on the first m - strip rows; with a stream-K plan
// (decided by pick, whose workspace size pick has checked) the last round's
// tiles are shared through ws.  The last `strip` rows go to the strip kernel.
template <typename T>
int run(const Variant<T>& v, int m, int n, int k, T alpha, const T* A, int lda, const T* B,
        int ldb, T beta, T* C, int ldc, const SkPlan& plan, T* ws, int strip, hipStream_t s) {
  if (ceil_div(m, v.bm) * ceil_div(n, v.bn) > kMaxTiles) return PGEMM_EHIP;
  GemmArgs<T> g{};
  if (plan.wgs > 0 && ws != nullptr) {
    g.full_tiles = plan.full_tiles;
    g.sk_wgs = plan.wgs;
    g.ws = ws;
  }
  g.M = m - strip;
  g.N = n;
  g.K = k;
  g.alpha = alpha;
  g.beta = beta;
  g.A = A;
  g.B = B;
  g.C = C;
  g.lda = lda;
  g.ldb = ldb;
  g.ldc = ldc;
  g.group_m = 4;
  int sc = 0;
  if (strip > 0) {
    v.strip_shape(strip, n, device_cus(), &sc, &g.strip_cgw);
    if (v.fstrip) g.strip_rows = strip;   // extra workgroups of the same grid
  }
  if (v.launch(g, s) != hipSuccess) return PGEMM_EHIP;
  if (strip > 0 && !v.fstrip) {
    g.M = m;
    int i0 = m - strip;
    void* args[] = {&g, &i0};
    if (hipLaunchKernel(reinterpret_cast<const void*>(&strip_rows_kernel<T>),
                        dim3((unsigned)ceil_div(n, (long long)sc * g.strip_cgw)),
                        dim3(kStripThreads), args, 0, s) !=
        hipSuccess)
      return PGEMM_EHIP;
  }
  return PGEMM_OK;
}

// Shared body of gemm_f32 / gemm_f64 and their forced-variant forms.
// forced < 0: choose; otherwise index into this precision's table.
template <typename T>
int gemm_impl(int forced, int m, int n, int k, T alpha, const T* A, int lda, const T* B,
              int ldb, T beta, T* C, int ldc, void* ws, size_t ws_bytes, void* stream) {
  const int st = check_args(m, n, k, alpha, A, lda, B, ldb, C, ldc);
  if (st != 0) return st;
  if (ws != nullptr && !aligned16(ws)) return -12;
  if (m == 0 || n == 0) return PGEMM_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (k == 0 || alpha == T(0))
    return launch_scale(m, n, beta, C, ldc, s) == hipSuccess ? PGEMM_OK : PGEMM_EHIP;
  const bool vec = vec_ok(A, lda, B, ldb, C, ldc);
  const Variant<T>* table;
  int count;
  if constexpr (sizeof(T) == 4) {
    table = tables().f32;
    count = tables().n32;
  } else {
    table = tables().f64;
    count = tables().n64;
  }
  int idx, strip = 0;
  SkPlan plan;
  if (forced >= 0) {
    if (forced >= count) return PGEMM_EVARIANT;
    idx = forced;
    if (table[idx].vec && !vec) return PGEMM_EVARIANT;
    if (table[idx].max_ldc > 0 && ldc > table[idx].max_ldc) return PGEMM_EVARIANT;
  } else {
    // stream-K only where pick chose it: a workspace too small for the
    // preferred plan gives exactly the plain entry point's launch, even if
    // the fallback tiling's own plan would fit
    idx = pick<T>(m, n, k, ldc, vec, ws != nullptr ? ws_bytes : 0, &plan, &strip);
  }
  return run(table[idx], m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, plan,
             static_cast<T*>(ws), strip, s);
}

// The scratch array of gemm_f32_noalloc: one copy per device, at its own
// address on each.  In host code `scratch` is only a stand-in for the
// device symbol; its device address comes from hipGetSymbolAddress, taken
// once per device with that device current and kept per device below.
static __device__ __align__(256) unsigned char scratch[PGEMM_SCRATCH_BYTES];

// Device address of `scratch` on the current device (nullptr if HIP cannot
// give it).
void* scratch_address() {
  static std::mutex mu;
  static void* ptrs[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (ptrs[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    ptrs[dev] = p;
  }
  return ptrs[dev];
}

// Workspace the stream-K path would use for this shape (0: none), for any
// ldc that every tile class takes.
template <typename T>
size_t workspace_impl(int m, int n, int k) {
  if (m <= 0 || n <= 0 || k <= 0) return 0;
  return choose<T>(m, n, k, true, 0).plan.bytes;
}

template <typename T>
int select_impl(int m, int n, int k, T alpha, const T* A, int lda, const T* B, int ldb,
                const T* C, int ldc, size_t ws_bytes, int* sk_wgs, int* strip_rows_out) {
  if (sk_wgs != nullptr) *sk_wgs = 0;
  if (strip_rows_out != nullptr) *strip_rows_out = 0;
  const int st = check_args(m, n, k, alpha, A, lda, B, ldb, C, ldc);
  if (st != 0) return st;
  if (m == 0 || n == 0 || k == 0 || alpha == T(0)) return 0;
  const bool vec = vec_ok(A, lda, B, ldb, C, ldc);
  SkPlan plan;
  int strip = 0;
  const int idx = pick<T>(m, n, k, ldc, vec, ws_bytes, &plan, &strip);
  if (sk_wgs != nullptr) *sk_wgs = plan.wgs;
  if (strip_rows_out != nullptr) *strip_rows_out = strip;
  if constexpr (sizeof(T) == 4) return 1 + idx;
  else return 1 + tables().n32 + idx;
}

}  // namespace
}  // namespace pgemm

using namespace pgemm;

extern "C" {

int gemm_f32(int m, int n, int k, float alpha, const float* A, int lda, const float* B,
             int ldb, float beta, float* C, int ldc, void* stream) {
  return gemm_impl<float>(-1, m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, nullptr, 0,
                          stream);
}

int gemm_f64(int m, int n, int k, double alpha, const double* A, int lda, const double* B,
             int ldb, double beta, double* C, int ldc, void* stream) {
  return gemm_impl<double>(-1, m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, nullptr, 0,
                           stream);
}

int gemm_f32_ws(int m, int n, int k, float alpha, const float* A, int lda, const float* B,
                int ldb, float beta, float* C, int ldc, void* workspace,
                size_t workspace_bytes, void* stream) {
  return gemm_impl<float>(-1, m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, workspace,
                          workspace_bytes, stream);
}

int gemm_f64_ws(int m, int n, int k, double alpha, const double* A, int lda,
                const double* B, int ldb, double beta, double* C, int ldc, void* workspace,
                size_t workspace_bytes, void* stream) {
  return gemm_impl<double>(-1, m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, workspace,
                           workspace_bytes, stream);
}

// gemm_f32_ws on the library's scratch array.  Any workspace of at least
// the shape's own need gives gemm_f32_ws the same plan, so passing the
// array's full size reproduces gemm_f32_ws with pgemm_workspace_f32 bytes.
int gemm_f32_noalloc(int m, int n, int k, float alpha, const float* A, int lda,
                     const float* B, int ldb, float beta, float* C, int ldc, void* stream) {
  const int st = check_args(m, n, k, alpha, A, lda, B, ldb, C, ldc);
  if (st != 0) return st;
  if (m == 0 || n == 0) return PGEMM_OK;
  if (workspace_impl<float>(m, n, k) > PGEMM_SCRATCH_BYTES) return PGEMM_ESCRATCH;
  void* ws = scratch_address();
  if (ws == nullptr) return PGEMM_EHIP;
  return gemm_impl<float>(-1, m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, ws,
                          PGEMM_SCRATCH_BYTES, stream);
}

size_t pgemm_workspace_f32(int m, int n, int k) { return workspace_impl<float>(m, n, k); }

size_t pgemm_workspace_f64(int m, int n, int k) { return workspace_impl<double>(m, n, k); }

// Row-major X (r x c, ld) is the column-major storage of X^T (c x r, ld), so
// C^T = B^T A^T is a column-major GEMM with m = N3, n = N1, k = N2.
int matmat_f64(int lda, int ldb, int ldc, const double* A, const double* B, double* C,
               int N1, int N2, int N3, void* stream) {
  const bool touch_c = N1 > 0 && N3 > 0;
  const bool read_ab = touch_c && N2 > 0;
  if (lda < (N2 > 1 ? N2 : 1)) return -1;
  if (ldb < (N3 > 1 ? N3 : 1)) return -2;
  if (ldc < (N3 > 1 ? N3 : 1)) return -3;
  if (read_ab && (A == nullptr || !elem_aligned(A))) return -4;
  if (read_ab && (B == nullptr || !elem_aligned(B))) return -5;
  if (touch_c && (C == nullptr || !elem_aligned(C))) return -6;
  if (N1 < 0) return -7;
  if (N2 < 0) return -8;
  if (N3 < 0) return -9;
  return gemm_f64(N3, N1, N2, 1.0, B, ldb, A, lda, 1.0, C, ldc, stream);
}

// Device copies of the host operands live in the caller's workspace with
// the caller's leading dimensions: each is one flat copy of the strided
// block (rows of ld elements, the last row N columns long), which moves
// pageable memory about 8x faster than a pitched copy (MI355X, 4096 x 4096
// fp64: 4.7 ms against 39.5 ms).  Blocks start on 256-byte boundaries.
static size_t block_elems(int rows, int cols, int ld) {
  return rows <= 0 || cols <= 0 ? 0 : (size_t)(rows - 1) * (size_t)ld + (size_t)cols;
}
static size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }

size_t pgemm_matmat_host_workspace(int lda, int ldb, int ldc, int N1, int N2, int N3) {
  if (N1 <= 0 || N2 <= 0 || N3 <= 0 || lda < N2 || ldb < N3 || ldc < N3) return 0;
  return round256(block_elems(N1, N2, lda) * 8) + round256(block_elems(N2, N3, ldb) * 8) +
         round256(block_elems(N1, N3, ldc) * 8);
}

int matmat_f64_host(int lda, int ldb, int ldc, const double* A, const double* B, double* C,
                    int N1, int N2, int N3, void* workspace, size_t workspace_bytes,
                    void* stream) {
  const bool touch_c = N1 > 0 && N3 > 0;
  const bool read_ab = touch_c && N2 > 0;
  if (lda < (N2 > 1 ? N2 : 1)) return -1;
  if (ldb < (N3 > 1 ? N3 : 1)) return -2;
  if (ldc < (N3 > 1 ? N3 : 1)) return -3;
  if (read_ab && (A == nullptr || !elem_aligned(A))) return -4;
  if (read_ab && (B == nullptr || !elem_aligned(B))) return -5;
  if (touch_c && (C == nullptr || !elem_aligned(C))) return -6;
  if (N1 < 0) return -7;
  if (N2 < 0) return -8;
  if (N3 < 0) return -9;
  if (!read_ab) return PGEMM_OK;   // empty C, or C + A*B with N2 = 0: C unchanged
  const size_t need = pgemm_matmat_host_workspace(lda, ldb, ldc, N1, N2, N3);
  if (workspace == nullptr || !aligned16(static_cast<const char*>(workspace))) return -10;
  if (workspace_bytes < need) return -11;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const size_t na = block_elems(N1, N2, lda), nb = block_elems(N2, N3, ldb),
               nc = block_elems(N1, N3, ldc);
  char* base = static_cast<char*>(workspace);
  double* Ad = reinterpret_cast<double*>(base);
  double* Bd = reinterpret_cast<double*>(base + round256(na * 8));
  double* Cd = reinterpret_cast<double*>(base + round256(na * 8) + round256(nb * 8));
  // Flat copies of the strided blocks (the padding between rows is read,
  // never used); the lecture packs the rows into a host buffer instead.
  if (hipMemcpyAsync(Ad, A, na * 8, hipMemcpyHostToDevice, s) != hipSuccess ||
      hipMemcpyAsync(Bd, B, nb * 8, hipMemcpyHostToDevice, s) != hipSuccess ||
      hipMemcpyAsync(Cd, C, nc * 8, hipMemcpyHostToDevice, s) != hipSuccess)
    return PGEMM_EHIP;
  const int st = matmat_f64(lda, ldb, ldc, Ad, Bd, Cd, N1, N2, N3, stream);
  if (st != PGEMM_OK) return st;
  // C goes back row by row when its rows are padded (the padding is never
  // written), in one flat copy when they are not.
  const hipError_t e =
      (ldc == N3) ? hipMemcpyAsync(C, Cd, nc * 8, hipMemcpyDeviceToHost, s)
                  : hipMemcpy2DAsync(C, (size_t)ldc * 8, Cd, (size_t)ldc * 8, (size_t)N3 * 8,
                                     N1, hipMemcpyDeviceToHost, s);
  if (e != hipSuccess || hipStreamSynchronize(s) != hipSuccess) return PGEMM_EHIP;
  return PGEMM_OK;
}

const char* pgemm_status_string(int status) {
  switch (status) {
    case PGEMM_OK: return "success";
    case PGEMM_EHIP: return "HIP call failed (kernel launch, copy or synchronization)";
    case PGEMM_EVARIANT: return "unknown or inapplicable kernel variant";
    case PGEMM_ESCRATCH:
      return "the shape needs more stream-K scratch than the library's fixed array "
             "(PGEMM_SCRATCH_BYTES); call gemm_f32_ws with a workspace instead";
    default: break;
  }
  if (status < 0 && status >= -14) return "invalid argument (see the argument position)";
  return "unknown status";
}

int pgemm_select_f32(int m, int n, int k, float alpha, const float* A, int lda,
                     const float* B, int ldb, float beta, const float* C, int ldc) {
  (void)beta;
  return select_impl<float>(m, n, k, alpha, A, lda, B, ldb, C, ldc, 0, nullptr, nullptr);
}

int pgemm_select_f64(int m, int n, int k, double alpha, const double* A, int lda,
                     const double* B, int ldb, double beta, const double* C, int ldc) {
  (void)beta;
  return select_impl<double>(m, n, k, alpha, A, lda, B, ldb, C, ldc, 0, nullptr, nullptr);
}

int pgemm_select_ws_f32(int m, int n, int k, float alpha, const float* A, int lda,
                        const float* B, int ldb, float beta, const float* C, int ldc,
                        size_t ws_bytes, int* sk_wgs, int* strip_rows) {
  (void)beta;
  return select_impl<float>(m, n, k, alpha, A, lda, B, ldb, C, ldc, ws_bytes, sk_wgs,
                            strip_rows);
}

int pgemm_select_ws_f64(int m, int n, int k, double alpha, const double* A, int lda,
                        const double* B, int ldb, double beta, const double* C, int ldc,
                        size_t ws_bytes, int* sk_wgs, int* strip_rows) {
  (void)beta;
  return select_impl<double>(m, n, k, alpha, A, lda, B, ldb, C, ldc, ws_bytes, sk_wgs,
                             strip_rows);
}

int pgemm_num_variants(void) { return tables().n32 + tables().n64; }

int pgemm_device_info(int* cus, int* clock_khz) {
  if (cus == nullptr) return -1;
  if (clock_khz == nullptr) return -2;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return PGEMM_EHIP;
  if (hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipDeviceGetAttribute(clock_khz, hipDeviceAttributeClockRate, dev) != hipSuccess)
    return PGEMM_EHIP;
  return PGEMM_OK;
}

const char* pgemm_variant_name(int variant) {
  if (variant >= 1 && variant <= tables().n32) return tables().f32[variant - 1].name;
  const int j = variant - 1 - tables().n32;
  if (j >= 0 && j < tables().n64) return tables().f64[j].name;
  return nullptr;
}

int gemm_f32_variant(int variant, int m, int n, int k, float alpha, const float* A, int lda,
                     const float* B, int ldb, float beta, float* C, int ldc, void* stream) {
  if (variant < 1 || variant > tables().n32) return PGEMM_EVARIANT;
  return gemm_impl<float>(variant - 1, m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, nullptr,
                          0, stream);
}

int gemm_f64_variant(int variant, int m, int n, int k, double alpha, const double* A,
                     int lda, const double* B, int ldb, double beta, double* C, int ldc,
                     void* stream) {
  const int j = variant - 1 - tables().n32;
  if (j < 0 || j >= tables().n64) return PGEMM_EVARIANT;
  return gemm_impl<double>(j, m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, nullptr, 0,
                           stream);
}

}  // extern "C"
