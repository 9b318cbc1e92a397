// Matrix-core GEMM instantiations for bf16 inputs (all tile families and operand layouts).
#include "mfma.hpp"

namespace tgemm {

hipError_t launch_mfma_bf16(const GemmParams& p, int tile, bool a_mn, bool b_mn, hipStream_t s,
                            int ks) {
  return launch_mfma_dtype<BF16>(p, tile, a_mn, b_mn, s, ks);
}

}  // namespace tgemm
