// Matrix-core GEMM instantiations for E5M2 inputs (A E5M2, B E5M2; all tile families and
// operand layouts).
#include "mfma.hpp"

namespace tgemm {

hipError_t launch_mfma_e5m2(const GemmParams& p, int tile, bool a_mn, bool b_mn, hipStream_t s) {
  return launch_mfma_dtype<E5M2, E5M2, false>(p, tile, a_mn, b_mn, s);
}

}  // namespace tgemm
