// fp32 tile configurations (v_mfma_f32_32x32x2f32).
//
// Name: f32_<BM>x<BN>x<BK>_w<waves down>x<waves across>_s<LDS stages>[_k2]_<vec|ua>.
// "vec" needs 16-byte aligned pointers and leading dimensions that are
// multiples of 4; "ua" (unaligned) takes any element-aligned input and still
// moves 16 bytes per global access.
#include "variants.hpp"

namespace pgemm {

// Threads per workgroup, the width limits of a configuration's own strip
// workgroups (used where it computes strip rows in its grid; see strip_cols)
// and the largest ldc it takes (0: any).
#define PGEMM_STRIP_LIMITS(...) \
  threads_of<__VA_ARGS__>(), strip_scmax_of<__VA_ARGS__>(), strip_acc_of<__VA_ARGS__>(), \
      max_ldc_of<__VA_ARGS__>()

#define PGEMM_F32(BM, BN, BK, WM, WN, S, VEC, SUFFIX)                                        \
  {"f32_" #BM "x" #BN "x" #BK "_w" #WM "x" #WN "_s" #S "_" #SUFFIX, BM, BN, BK, VEC, false, false, \
   &launch_tile<TraitF32, BM, BN, BK, WM, WN, VEC, S>, \
   PGEMM_STRIP_LIMITS(TraitF32, BM, BN, BK, WM, WN, VEC, S)}
// The same with the stream-K form compiled in (the tile classes the shape
// choice uses) and with rows below the last whole tile row computed by extra
// workgroups of the same grid (these classes' LDS leaves room for a second
// workgroup per compute unit beside a tile).
#define PGEMM_F32_SK(BM, BN, BK, WM, WN, S, VEC, SUFFIX)                                    \
  {"f32_" #BM "x" #BN "x" #BK "_w" #WM "x" #WN "_s" #S "_" #SUFFIX, BM, BN, BK, VEC, true, true, \
   &launch_tile<TraitF32, BM, BN, BK, WM, WN, VEC, S, 1, true, true>, \
   PGEMM_STRIP_LIMITS(TraitF32, BM, BN, BK, WM, WN, VEC, S, 1)}
// _k2: two groups of WM x WN waves split each K tile's inner indices.
#define PGEMM_F32_K2(BM, BN, BK, WM, WN, S, VEC, SUFFIX)                                          \
  {"f32_" #BM "x" #BN "x" #BK "_w" #WM "x" #WN "_s" #S "_k2_" #SUFFIX, BM, BN, BK, VEC, false, false, \
   &launch_tile<TraitF32, BM, BN, BK, WM, WN, VEC, S, 2>, \
   PGEMM_STRIP_LIMITS(TraitF32, BM, BN, BK, WM, WN, VEC, S, 2)}
#define PGEMM_F32_K2_SK(BM, BN, BK, WM, WN, S, VEC, SUFFIX)                                      \
  {"f32_" #BM "x" #BN "x" #BK "_w" #WM "x" #WN "_s" #S "_k2_" #SUFFIX, BM, BN, BK, VEC, true, true, \
   &launch_tile<TraitF32, BM, BN, BK, WM, WN, VEC, S, 2, true, true>, \
   PGEMM_STRIP_LIMITS(TraitF32, BM, BN, BK, WM, WN, VEC, S, 2)}

// _k4: four groups of WM x WN waves split each K tile's inner indices.
#define PGEMM_F32_K4(BM, BN, BK, WM, WN, S, VEC, SUFFIX)                                          \
  {"f32_" #BM "x" #BN "x" #BK "_w" #WM "x" #WN "_s" #S "_k4_" #SUFFIX, BM, BN, BK, VEC, false, false, \
   &launch_tile<TraitF32, BM, BN, BK, WM, WN, VEC, S, 4>, \
   PGEMM_STRIP_LIMITS(TraitF32, BM, BN, BK, WM, WN, VEC, S, 4)}

// A host function owns the table so that it is never treated as device data.
const Variant<float>* f32_variants(int* count) {
  static const Variant<float> table[] = {
      // LDS ring of 3, 8 waves (2 per SIMD), wave tile 128 x 64: large
      // problems (no stream-K form: with its piece loop the 128 x 64 wave
      // tile no longer fits the registers)
      PGEMM_F32(256, 256, 16, 2, 4, 3, true, vec),
      PGEMM_F32(256, 256, 16, 2, 4, 3, false, ua),
      // 256 x 128 tiles, 8 waves of 64 x 64: shapes where whole rounds of
      // these tiles beat both neighbours
      PGEMM_F32(256, 128, 32, 4, 2, 3, true, vec),
      PGEMM_F32(256, 128, 32, 4, 2, 3, false, ua),
      // 128 x 128 tiles fill 256 CUs from 2048^2: K split over two groups
      // of 4 waves with 64 x 64 wave tiles, 8 waves of 32 x 64 with BK 32,
      // or (the 128 x 128 class: least fixed cost per tile) 8 waves of
      // 32 x 64 on a ring of 4 stages of BK 16
      PGEMM_F32_K2(128, 128, 32, 2, 2, 3, true, vec),
      PGEMM_F32_K2(128, 128, 32, 2, 2, 3, false, ua),
      PGEMM_F32(128, 128, 32, 4, 2, 3, true, vec),
      PGEMM_F32(128, 128, 32, 4, 2, 3, false, ua),
      PGEMM_F32_SK(128, 128, 16, 4, 2, 4, true, vec),
      PGEMM_F32_SK(128, 128, 16, 4, 2, 4, false, ua),
      // ring, 4 waves (1 per SIMD)
      PGEMM_F32(256, 256, 16, 2, 2, 3, true, vec),     // wave tile 128 x 128
      PGEMM_F32(128, 128, 16, 2, 2, 4, true, vec),     // wave tile 64 x 64
      // plain double buffering (two LDS stages), 4 waves
      PGEMM_F32(128, 128, 32, 2, 2, 2, true, vec),
      PGEMM_F32(128, 128, 32, 2, 2, 2, false, ua),
      // 64 x 64 tiles, 4 waves of 32 x 32 on a ring of 4 stages of BK 16:
      // 256 tiles from 1024^2, and 32 KiB of LDS and ~50 VGPRs, so several
      // workgroups share a compute unit when there are more tiles than units
      PGEMM_F32_SK(64, 64, 16, 2, 2, 4, true, vec),
      PGEMM_F32_SK(64, 64, 16, 2, 2, 4, false, ua),
      // 64 x 64 tiles with two K groups of 4 waves (8 waves, two per SIMD)
      // on a ring of 3 stages of BK 32: long K loops on few tiles per
      // compute unit, where one wave per SIMD cannot hide the memory latency
      PGEMM_F32_K2_SK(64, 64, 32, 2, 2, 3, true, vec),
      PGEMM_F32_K2_SK(64, 64, 32, 2, 2, 3, false, ua),
      // 32 x 32 tiles, four K groups of one wave (one per SIMD); and 64 x 64
      // tiles, four K groups of 4 waves (16 waves, four per SIMD): small
      // problems, where tiles per compute unit, not operand traffic, decide
      PGEMM_F32_K4(32, 32, 64, 1, 1, 3, true, vec),
      PGEMM_F32_K4(32, 32, 64, 1, 1, 3, false, ua),
      PGEMM_F32_K4(64, 64, 64, 2, 2, 3, true, vec),
      PGEMM_F32_K4(64, 64, 64, 2, 2, 3, false, ua),
  };
  *count = (int)(sizeof(table) / sizeof(table[0]));
  return table;
}

}  // namespace pgemm
