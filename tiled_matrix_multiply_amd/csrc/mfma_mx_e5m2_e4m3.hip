// Matrix-core GEMM instantiations for block-scaled (MX) E5M2 x E4M3 inputs (A E5M2, B E4M3; all tile families and
// operand layouts).
#include "mfma.hpp"

namespace tgemm {

hipError_t launch_mfma_mx_e5m2_e4m3(const GemmParams& p, int tile, bool a_mn, bool b_mn, hipStream_t s) {
  return launch_mfma_dtype<E5M2, E4M3, true>(p, tile, a_mn, b_mn, s);
}

}  // namespace tgemm
