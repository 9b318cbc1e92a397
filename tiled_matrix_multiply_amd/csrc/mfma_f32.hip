// Matrix-core GEMM instantiations for f32 inputs (all tile families and operand layouts).
#include "mfma.hpp"

namespace tgemm {

hipError_t launch_mfma_f32(const GemmParams& p, int tile, bool a_mn, bool b_mn, hipStream_t s,
                           int ks) {
  return launch_mfma_dtype<F32>(p, tile, a_mn, b_mn, s, ks);
}

}  // namespace tgemm
