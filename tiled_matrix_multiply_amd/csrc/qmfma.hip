// Placeholder replaced by the matrix-core quantized kernel.
#include "quant.hpp"
namespace tgemm {
hipError_t launch_qmfma(const QParams&, int, hipStream_t) { return hipErrorNotSupported; }
}  // namespace tgemm
