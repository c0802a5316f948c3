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
  LaunchFn<T> launch;
};

// Launch one tile configuration.  Plain: one workgroup per BM x BN tile of
// C.  Split (a.split > 1): one workgroup per tile for the first a.full_tiles
// tiles and a.split workgroups (K slices writing partial sums to a.ws) for
// each remaining tile, then the fix-up kernel.
template <class TR, int BM, int BN, int BK, int WGM, int WGN, bool VEC, int STAGES, int KS = 1>
hipError_t launch_tile(const GemmArgs<typename TR::T>& a, hipStream_t stream) {
  using T = typename TR::T;
  GemmArgs<T> g = a;
  g.tiles_m = (g.M + BM - 1) / BM;
  g.tiles_n = (g.N + BN - 1) / BN;
  const int tiles = g.tiles_m * g.tiles_n;
  if (g.group_m <= 0) g.group_m = 4;
  if (g.split <= 1 || g.ws == nullptr || g.full_tiles >= tiles) {
    g.full_tiles = tiles;
    g.split = 1;
  }
  const int rest = tiles - g.full_tiles;
  g.buf32 = buffer_offsets_fit<T>(BM, BN, BK, g.lda, g.ldb) ? 1 : 0;
  void* args[] = {&g};
  const dim3 grid((unsigned)(g.full_tiles + rest * g.split)), block(WGM * WGN * 64 * KS);
  hipError_t e = hipLaunchKernel(
      reinterpret_cast<const void*>(&gemm_tile_kernel<TR, BM, BN, BK, WGM, WGN, VEC, STAGES, KS>),
      grid, block, args, 0, stream);
  if (e != hipSuccess || rest == 0) return e;
  int bm = BM, bn = BN;
  void* fargs[] = {&g, &bm, &bn};
  return hipLaunchKernel(reinterpret_cast<const void*>(&split_fixup_kernel<T>),
                         dim3((unsigned)((BM * BN + 255) / 256), (unsigned)rest), dim3(256),
                         fargs, 0, stream);
}

// The compiled configurations of each precision, in a fixed order.
const Variant<float>* f32_variants(int* count);
const Variant<double>* f64_variants(int* count);

}  // namespace pgemm
