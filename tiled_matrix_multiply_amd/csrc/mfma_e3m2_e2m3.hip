// Matrix-core GEMM instantiations for packed 6-bit inputs, A E3M2 and B E2M3 (OCP MX 6-bit
// floats), per-tensor and block-scaled (MX).  Packed operands are staged K-contiguous only: A
// stored M x K, B stored N x K.
#include "mfma.hpp"

namespace tgemm {

hipError_t launch_mfma_e3m2_e2m3(const GemmParams& p, int tile, bool a_mn, bool b_mn, hipStream_t s) {
  return launch_mfma_dtype<E3M2, E2M3, false>(p, tile, a_mn, b_mn, s);
}

hipError_t launch_mfma_mx_e3m2_e2m3(const GemmParams& p, int tile, bool a_mn, bool b_mn, hipStream_t s) {
  return launch_mfma_dtype<E3M2, E2M3, true>(p, tile, a_mn, b_mn, s);
}

}  // namespace tgemm
