// The decomposed epilogue: C = GELU(C + bias) (either part optional) as its own elementwise
// pass over an M x N matrix already written by a GEMM without epilogue.  This is the unfused
// path that "Rigel" (arXiv 2606.12765) compares its fused GEMM + bias + GELU against (abstract;
// section 1, contribution 7).  It is bound by HBM: it reads and writes every element once.
#include "common.hpp"

namespace tgemm {

// Vector path: each thread handles 8 consecutive elements of one row (16 bytes of a 16-bit C,
// 32 bytes of fp32 C); requires N % 8 == 0, ldc % 8 == 0 and a 16-byte-aligned C.
template <int CT>
__global__ __launch_bounds__(256) void bias_gelu_vec_kernel(void* C, int64_t ldc, int M, int N,
                                                            const float* bias, uint32_t epi) {
  const int per_row = N / 8;
  const int64_t total = (int64_t)M * per_row;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int m = (int)(t / per_row), n = (int)(t % per_row) * 8;
    const int64_t idx = (int64_t)m * ldc + n;
    float v[8];
    if constexpr (CT == F32) {
      const float4* src = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(C) + idx);
      const float4 a = src[0], b = src[1];
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
      const uint4 w = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(C) + idx);
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t h = (ws[e >> 1] >> ((e & 1) * 16)) & 0xffffu;
        v[e] = (CT == F16) ? f16_bits_to_float(h) : bf16_bits_to_float(h);
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = v[e];
      if (epi & EPI_BIAS) x += bias[n + e];
      if (epi & EPI_GELU) x = gelu_out<CT>(x);
      v[e] = x;
    }
    if constexpr (CT == F32) {
      float4* dst = reinterpret_cast<float4*>(reinterpret_cast<float*>(C) + idx);
      dst[0] = float4{v[0], v[1], v[2], v[3]};
      dst[1] = float4{v[4], v[5], v[6], v[7]};
    } else {
      uint32_t h[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) h[e] = (CT == F16) ? float_to_f16_bits(v[e]) : float_to_bf16_bits(v[e]);
      *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(C) + idx) =
          uint4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
    }
  }
}

// Scalar path for any alignment.
template <int CT>
__global__ __launch_bounds__(256) void bias_gelu_scalar_kernel(void* C, int64_t ldc, int M, int N,
                                                               const float* bias, uint32_t epi) {
  const int64_t total = (int64_t)M * N;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int m = (int)(t / N), n = (int)(t % N);
    const int64_t idx = (int64_t)m * ldc + n;
    float x = load_as_float<CT>(C, idx);
    if (epi & EPI_BIAS) x += bias[n];
    if (epi & EPI_GELU) x = gelu_out<CT>(x);
    store_from_float<CT>(C, idx, x);
  }
}

template <int CT>
static hipError_t launch_ct(void* C, int64_t ldc, int M, int N, const float* bias, uint32_t epi,
                            bool vec, int cu_count, hipStream_t s) {
  const int64_t items = vec ? (int64_t)M * (N / 8) : (int64_t)M * N;
  const int64_t want = (items + 255) / 256;
  const int64_t cap = (int64_t)cu_count * 16;  // enough resident waves to saturate HBM
  const unsigned grid = (unsigned)(want < cap ? (want > 0 ? want : 1) : cap);
  if (vec)
    hipLaunchKernelGGL((bias_gelu_vec_kernel<CT>), dim3(grid), dim3(256), 0, s, C, ldc, M, N, bias, epi);
  else
    hipLaunchKernelGGL((bias_gelu_scalar_kernel<CT>), dim3(grid), dim3(256), 0, s, C, ldc, M, N, bias, epi);
  return hipGetLastError();
}

hipError_t launch_bias_gelu(void* C, int64_t ldc, int M, int N, int c_type, const float* bias,
                            uint32_t epi, int cu_count, hipStream_t s) {
  const bool vec = (N % 8 == 0) && (ldc % 8 == 0) && ((reinterpret_cast<uintptr_t>(C) & 15) == 0);
  switch (c_type) {
    case F32: return launch_ct<F32>(C, ldc, M, N, bias, epi, vec, cu_count, s);
    case F16: return launch_ct<F16>(C, ldc, M, N, bias, epi, vec, cu_count, s);
    case BF16: return launch_ct<BF16>(C, ldc, M, N, bias, epi, vec, cu_count, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tgemm
