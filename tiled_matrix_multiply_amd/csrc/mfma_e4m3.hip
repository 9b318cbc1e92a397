// Matrix-core GEMM instantiations for E4M3 inputs (A E4M3, B E4M3; all tile families and
// operand layouts).
#include "mfma.hpp"

namespace tgemm {

hipError_t launch_mfma_e4m3(const GemmParams& p, int tile, bool a_mn, bool b_mn, hipStream_t s) {
  return launch_mfma_dtype<E4M3, E4M3, false>(p, tile, a_mn, b_mn, s);
}

}  // namespace tgemm
