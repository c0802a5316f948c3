// fp32 tile configurations (v_mfma_f32_32x32x2f32).
#include "variants.hpp"

namespace pgemm {

#define PGEMM_F32(BM, BN, BK, WM, WN, VEC, SUFFIX)                       \
  {"f32_" #BM "x" #BN "x" #BK "_w" #WM "x" #WN "_" #SUFFIX, BM, BN, BK, VEC, \
   &launch_tile<TraitF32, BM, BN, BK, WM, WN, VEC>}

// A host function owns the table so that it is never treated as device data.
const Variant<float>* f32_variants(int* count) {
  static const Variant<float> table[] = {
      PGEMM_F32(256, 256, 32, 2, 2, true, vec),   // wave tile 128 x 128
      PGEMM_F32(256, 256, 32, 2, 2, false, scalar),
      PGEMM_F32(256, 256, 16, 2, 2, true, vec),
      PGEMM_F32(256, 256, 16, 2, 2, false, scalar),
      PGEMM_F32(128, 128, 32, 2, 2, true, vec),   // wave tile 64 x 64
      PGEMM_F32(128, 128, 32, 2, 2, false, scalar),
      PGEMM_F32(256, 128, 32, 2, 2, true, vec),   // wave tile 128 x 64
      PGEMM_F32(256, 128, 32, 2, 2, false, scalar),
  };
  *count = (int)(sizeof(table) / sizeof(table[0]));
  return table;
}

}  // namespace pgemm
