// fp64 tile configurations (v_mfma_f64_16x16x4f64).
//
// Name: f64_<BM>x<BN>x<BK>_w<waves down>x<waves across>_s<LDS stages>_<vec|ua>.
// "vec" needs 16-byte aligned pointers and even leading dimensions; "ua"
// (unaligned) takes any element-aligned input and still moves 16 bytes per
// global access.
#include "variants.hpp"

namespace pgemm {

// Threads per workgroup, the width limits of a configuration's own strip
// workgroups (used where it computes strip rows in its grid; see strip_cols)
// and the largest ldc it takes (0: any).
#define PGEMM_STRIP_LIMITS(...) \
  threads_of<__VA_ARGS__>(), strip_scmax_of<__VA_ARGS__>(), strip_acc_of<__VA_ARGS__>(), \
      max_ldc_of<__VA_ARGS__>()

#define PGEMM_F64(BM, BN, BK, WM, WN, S, VEC, SUFFIX)                                        \
  {"f64_" #BM "x" #BN "x" #BK "_w" #WM "x" #WN "_s" #S "_" #SUFFIX, BM, BN, BK, VEC, false, false, \
   &launch_tile<TraitF64, BM, BN, BK, WM, WN, VEC, S>, \
   PGEMM_STRIP_LIMITS(TraitF64, BM, BN, BK, WM, WN, VEC, S)}
// The same with the stream-K form compiled in (the tile classes the shape
// choice uses); FS: rows below the last whole tile row are computed by extra
// workgroups of the same grid (classes whose LDS leaves room for a second
// workgroup per compute unit), otherwise by the strip kernel after it.
#define PGEMM_F64_SK(BM, BN, BK, WM, WN, S, VEC, SUFFIX, FS)                                \
  {"f64_" #BM "x" #BN "x" #BK "_w" #WM "x" #WN "_s" #S "_" #SUFFIX, BM, BN, BK, VEC, true, FS, \
   &launch_tile<TraitF64, BM, BN, BK, WM, WN, VEC, S, 1, true, FS>, \
   PGEMM_STRIP_LIMITS(TraitF64, BM, BN, BK, WM, WN, VEC, S, 1)}

// A host function owns the table so that it is never treated as device data.
const Variant<double>* f64_variants(int* count) {
  static const Variant<double> table[] = {
      // LDS ring of 3, 8 waves, wave tile 64 x 32, unrolled steady state:
      // the large-problem class
      PGEMM_F64_SK(128, 128, 16, 2, 4, 3, true, vec, false),
      PGEMM_F64_SK(128, 128, 16, 2, 4, 3, false, ua, false),
      // LDS ring of 3, 8 waves, wave tile 64 x 64 (too many registers to
      // unroll the steady state)
      PGEMM_F64(256, 128, 16, 4, 2, 3, true, vec),
      PGEMM_F64(256, 128, 16, 4, 2, 3, false, ua),
      // plain double buffering
      PGEMM_F64(256, 128, 16, 2, 4, 2, true, vec),
      PGEMM_F64(128, 128, 16, 2, 2, 2, true, vec),
      PGEMM_F64(128, 128, 16, 2, 2, 2, false, ua),
      // 64 x 64 tiles, 8 waves of 32 x 16 on a ring of 4 (2048^3: 72.0
      // TFLOP/s against 61.3 on a ring of 3): shapes whose 128 x 128 tiles
      // leave a badly filled last round, and small ones
      PGEMM_F64_SK(64, 64, 16, 2, 4, 4, true, vec, true),
      PGEMM_F64_SK(64, 64, 16, 2, 4, 4, false, ua, true),
  };
  *count = (int)(sizeof(table) / sizeof(table[0]));
  return table;
}

}  // namespace pgemm
