// Internal: the compiled tile configurations of each precision.
#pragma once

#include <hip/hip_runtime.h>

#include "gemm_tile.hpp"

namespace pgemm {

template <typename T>
using LaunchFn = hipError_t (*)(const GemmArgs<T>&, hipStream_t);

template <typename T>
struct Variant {
  const char* name;
  int bm, bn, bk;
  bool vec;        // needs 16-byte aligned pointers and leading dims
  bool sk;         // has the stream-K form
  bool fstrip;     // computes strip rows in extra workgroups of its own grid
  LaunchFn<T> launch;
  int threads;     // per workgroup
  int strip_scmax, strip_acc;   // the grid's own strip role (see strip_cols)
  long long max_ldc;   // largest ldc the configuration takes (0: any; see TileCfg::WT_MAX_LDC)
  // Columns per wave and column groups per workgroup of the strip of r rows
  // over n columns on `units` compute units: the grid's own strip role, or
  // the strip kernel's.
  void strip_shape(int r, int n, int units, int* sc, int* cgw) const {
    const int nt = fstrip ? threads : kStripThreads;
    *sc = fstrip ? pgemm::strip_cols(r, strip_scmax, strip_acc)
                 : pgemm::strip_cols(r, strip_kernel_scmax<T>(), strip_kernel_acc<T>());
    *cgw = strip_groups(n, *sc, nt / 64, units);
  }
};

// Threads and strip limits of a tile configuration, for its Variant entry.
template <class TR, int BM, int BN, int BK, int WGM, int WGN, bool VEC, int STAGES, int KS = 1>
constexpr int threads_of() {
  return TileCfg<TR, BM, BN, BK, WGM, WGN, VEC, STAGES, KS>::NT;
}
template <class TR, int BM, int BN, int BK, int WGM, int WGN, bool VEC, int STAGES, int KS = 1>
constexpr int strip_scmax_of() {
  return TileCfg<TR, BM, BN, BK, WGM, WGN, VEC, STAGES, KS>::STRIP_SCMAX;
}
template <class TR, int BM, int BN, int BK, int WGM, int WGN, bool VEC, int STAGES, int KS = 1>
constexpr int strip_acc_of() {
  return TileCfg<TR, BM, BN, BK, WGM, WGN, VEC, STAGES, KS>::STRIP_ACC;
}
template <class TR, int BM, int BN, int BK, int WGM, int WGN, bool VEC, int STAGES, int KS = 1>
constexpr long long max_ldc_of() {
  return TileCfg<TR, BM, BN, BK, WGM, WGN, VEC, STAGES, KS>::WT_MAX_LDC;
}

// Launch one tile configuration.  Plain: one workgroup per BM x BN tile of
// C.  Stream-K (SK compiled in, a.sk_wgs > 0 with a workspace): one
// workgroup per tile for the first a.full_tiles tiles, a.sk_wgs workgroups
// that share the K tiles of the remaining ones (partial sums to a.ws), then
// the fix-up kernel.  Without SK a stream-K request runs plain.  Strip rows
// (FS compiled in, a.strip_rows > 0): a.strip_wgs more workgroups at the
// end of the grid compute rows [a.M, a.M + a.strip_rows); without FS they
// are ignored here (the caller launches the strip kernel).
template <class TR, int BM, int BN, int BK, int WGM, int WGN, bool VEC, int STAGES, int KS = 1,
          bool SK = false, bool FS = false>
hipError_t launch_tile(const GemmArgs<typename TR::T>& a, hipStream_t stream) {
  using T = typename TR::T;
  GemmArgs<T> g = a;
  g.tiles_m = (g.M + BM - 1) / BM;
  g.tiles_n = (g.N + BN - 1) / BN;
  const int tiles = g.tiles_m * g.tiles_n;
  if (g.group_m <= 0) g.group_m = 4;
  if (!SK || g.sk_wgs <= 0 || g.ws == nullptr || g.full_tiles >= tiles) {
    g.full_tiles = tiles;
    g.sk_wgs = 0;
  }
  const bool strip = FS && g.strip_rows > 0 && g.strip_cgw > 0;
  if (strip) {
    using Cfg = TileCfg<TR, BM, BN, BK, WGM, WGN, VEC, STAGES, KS>;
    const int sc = strip_cols(g.strip_rows, Cfg::STRIP_SCMAX, Cfg::STRIP_ACC);
    g.strip_wgs = (g.N + g.strip_cgw * sc - 1) / (g.strip_cgw * sc);
  } else {
    g.strip_rows = 0;
    g.strip_wgs = 0;
  }
  const int rest = tiles - g.full_tiles;
  {
    using Cfg = TileCfg<TR, BM, BN, BK, WGM, WGN, VEC, STAGES, KS>;
    // stores of C with 32-bit offsets from the tile's first element
    if (Cfg::WT_MAX_LDC > 0 && g.ldc > Cfg::WT_MAX_LDC) return hipErrorInvalidValue;
  }
  g.buf32 = buffer_offsets_fit<T>(BM, BN, BK, g.lda, g.ldb) ? 1 : 0;
  void* args[] = {&g};
  const dim3 grid((unsigned)(g.full_tiles + g.sk_wgs + g.strip_wgs)),
      block(WGM * WGN * 64 * KS);
  const void* kern;
  if (rest == 0)
    kern = strip ? reinterpret_cast<const void*>(
                       &gemm_tile_kernel<TR, BM, BN, BK, WGM, WGN, VEC, STAGES, KS, false, FS>)
                 : reinterpret_cast<const void*>(
                       &gemm_tile_kernel<TR, BM, BN, BK, WGM, WGN, VEC, STAGES, KS, false>);
  else
    kern = strip ? reinterpret_cast<const void*>(
                       &gemm_tile_kernel<TR, BM, BN, BK, WGM, WGN, VEC, STAGES, KS, SK, FS>)
                 : reinterpret_cast<const void*>(
                       &gemm_tile_kernel<TR, BM, BN, BK, WGM, WGN, VEC, STAGES, KS, SK>);
  hipError_t e = hipLaunchKernel(kern, grid, block, args, 0, stream);
  if (e != hipSuccess || rest == 0) return e;
  int bm = BM, bn = BN, bk = BK;
  void* fargs[] = {&g, &bm, &bn, &bk};
  return hipLaunchKernel(reinterpret_cast<const void*>(&sk_fixup_kernel<T>),
                         dim3((unsigned)((BM * BN + 255) / 256), (unsigned)rest), dim3(256),
                         fargs, 0, stream);
}

// The compiled configurations of each precision, in a fixed order.
const Variant<float>* f32_variants(int* count);
const Variant<double>* f64_variants(int* count);

}  // namespace pgemm
