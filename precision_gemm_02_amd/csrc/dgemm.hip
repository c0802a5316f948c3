// fp64 tile configurations (v_mfma_f64_16x16x4f64).
#include "variants.hpp"

namespace pgemm {

#define PGEMM_F64(BM, BN, BK, WM, WN, VEC, SUFFIX)                       \
  {"f64_" #BM "x" #BN "x" #BK "_w" #WM "x" #WN "_" #SUFFIX, BM, BN, BK, VEC, \
   &launch_tile<TraitF64, BM, BN, BK, WM, WN, VEC>}

// A host function owns the table so that it is never treated as device data.
const Variant<double>* f64_variants(int* count) {
  static const Variant<double> table[] = {
      PGEMM_F64(128, 128, 16, 2, 2, true, vec),   // wave tile 64 x 64
      PGEMM_F64(128, 128, 16, 2, 2, false, scalar),
      PGEMM_F64(128, 128, 32, 2, 2, true, vec),
      PGEMM_F64(128, 128, 32, 2, 2, false, scalar),
  };
  *count = (int)(sizeof(table) / sizeof(table[0]));
  return table;
}

}  // namespace pgemm
