// Matrix-core kernel for group-quantized weights (prefill): the tiled MFMA kernel with its B
// operand staged from codes, dequantised in registers and written to LDS as 16-bit values.
#include "mfma.hpp"
#include "quant.hpp"

namespace tgemm {

template <int DT, int QB, int TILE, int WM, int WN>
hipError_t launch_qmfma_cfg(const GemmParams& p, hipStream_t s) {
  return launch_mfma_cfg<MfmaCfg<DT, TILE, WM, WN, false, false, 2, DT, false, QB>>(p, s);
}

template <int DT, int QB>
hipError_t launch_qmfma_tile(GemmParams p, int cu_count, hipStream_t s) {
  auto tiles = [&](int t) { return (int64_t)((p.M + t - 1) / t) * ((p.N + t - 1) / t); };
  // the 256 x 256 tile when it still gives every compute unit a workgroup, else 128 x 128
  // (prefill shapes are large; few activation rows go to the matrix-vector kernel)
  if (tiles(256) >= cu_count) {
    p.tiles_m = (p.M + 255) / 256;
    p.tiles_n = (p.N + 255) / 256;
    return launch_qmfma_cfg<DT, QB, 256, 2, 4>(p, s);
  }
  p.tiles_m = (p.M + 127) / 128;
  p.tiles_n = (p.N + 127) / 128;
  return launch_qmfma_cfg<DT, QB, 128, 2, 2>(p, s);
}

// The host has checked: 16-byte aligned X, codes and C; ldx a multiple of 8, ldw of 16, ldc of
// 4; group a multiple of 32 and K a multiple of 64 (whole K tiles, each thread's 32 codes in
// one group).
hipError_t launch_qmfma(const QParams& q, int x_type, int cu_count, hipStream_t s) {
  GemmParams p{};
  p.A = q.X;
  p.B = q.W;
  p.C = q.C;
  p.bias = q.bias;
  p.lda = q.ldx;
  p.ldb = q.ldw;  // bytes
  p.ldc = q.ldc;
  p.M = q.M;
  p.N = q.N;
  p.K = q.K;
  p.alpha = q.alpha;
  p.beta = q.beta;
  p.epi = q.epi;
  p.qs = q.S;
  p.qo = q.O;
  p.ldg = q.ldg;
  p.group = q.group;
  if (x_type == BF16)
    return q.bits == 4 ? launch_qmfma_tile<BF16, 4>(p, cu_count, s) : launch_qmfma_tile<BF16, 8>(p, cu_count, s);
  return q.bits == 4 ? launch_qmfma_tile<F16, 4>(p, cu_count, s) : launch_qmfma_tile<F16, 8>(p, cu_count, s);
}

}  // namespace tgemm
