// The decomposed epilogue: C = GELU(C + bias) (either part optional) as its own elementwise
// pass over an M x N matrix already written by a GEMM without epilogue.  This is the unfused
// path that "Rigel" (arXiv 2606.12765) compares its fused GEMM + bias + GELU against (abstract;
// section 1, contribution 7).  It is bound by HBM: it reads and writes every element once.
#include "common.hpp"

namespace tgemm {

// Vector path: a workgroup is TX x (256 / TX) threads.  Thread (x, y) of workgroup (bx, by)
// owns the 8 consecutive elements of column chunk c = TX bx + x (16 bytes of a 16-bit C, 32 of
// fp32 C) in the R rows R (by (256 / TX) + y) ..  + R-1, then the rows gridDim.y (256 / TX) R
// further on.  Its R loads are issued before any GELU, so each thread keeps R reads in flight,
// and no index is divided.  The chunk's bias values are read once.  Requires N % 8 == 0,
// ldc % 8 == 0 and a 16-byte-aligned C.
// For 16-bit outputs with GELU the elementwise work is the fused epilogue's: y = (x + b) / 2
// (one fma with the bias halved; halving is exact) and gelu16_half(y).
template <int CT, int R>
__global__ __launch_bounds__(256) void bias_gelu_vec_kernel(void* C, int64_t ldc, int M, int N,
                                                            const float* bias, uint32_t epi, int TX) {
  const int ty = threadIdx.x / TX, tx = threadIdx.x % TX, TY = 256 / TX;
  const int c = blockIdx.x * TX + tx;
  if (c >= N / 8) return;
  const int n = 8 * c;
  const bool half = CT != F32 && (epi & EPI_GELU);
  const float hs = half ? 0.5f : 1.0f;
  float bj[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) bj[e] = (epi & EPI_BIAS) ? hs * bias[n + e] : 0.0f;
  typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
  for (int64_t m0 = ((int64_t)blockIdx.y * TY + ty) * R; m0 < M; m0 += (int64_t)gridDim.y * TY * R) {
    u32x8 w[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (m0 + r >= M) break;
      const int64_t idx = (m0 + r) * ldc + n;
      if constexpr (CT == F32) {
        const uint4* src = reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(C) + idx);
        const uint4 a = src[0], b = src[1];
        w[r] = u32x8{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
      } else {
        const uint4 h = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(C) + idx);
        w[r] = u32x8{h.x, h.y, h.z, h.w, 0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (m0 + r >= M) break;
      const int64_t idx = (m0 + r) * ldc + n;
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float x;
        if constexpr (CT == F32) {
          x = __uint_as_float(w[r][e]);
        } else {
          const uint32_t h = (w[r][e >> 1] >> ((e & 1) * 16)) & 0xffffu;
          x = (CT == F16) ? f16_bits_to_float(h) : bf16_bits_to_float(h);
        }
        if (half) {
          v[e] = gelu16_half(fmaf(0.5f, x, bj[e]));
        } else {
          x += bj[e];
          if (epi & EPI_GELU) x = gelu_out<CT>(x);
          v[e] = x;
        }
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
  if (vec) {
    // TX threads across the row's chunks (a power of two from 64 to 256), 256 / TX rows; R = 4
    // rows per thread once the pass has 2048 chunks per compute unit (a full complement of
    // resident threads), 2 from half that, else one: small passes want every chunk in its own
    // thread, large ones several loads in flight per thread (bf16 2048^2: 9 -> 6 us with 4).
    const int chunks = N / 8;
    int tx = 64;
    while (tx < 256 && tx < chunks) tx *= 2;
    const int64_t items = (int64_t)M * chunks, full = (int64_t)cu_count * 2048;
    const int r = items >= full ? 4 : items >= full / 2 ? 2 : 1;
    const unsigned gx = (unsigned)((chunks + tx - 1) / tx);
    const int64_t gy = ((int64_t)M + (int64_t)(256 / tx) * r - 1) / ((int64_t)(256 / tx) * r);
    const dim3 grid(gx, (unsigned)(gy < 65535 ? gy : 65535));
    if (r == 4)
      hipLaunchKernelGGL((bias_gelu_vec_kernel<CT, 4>), grid, dim3(256), 0, s, C, ldc, M, N, bias, epi, tx);
    else if (r == 2)
      hipLaunchKernelGGL((bias_gelu_vec_kernel<CT, 2>), grid, dim3(256), 0, s, C, ldc, M, N, bias, epi, tx);
    else
      hipLaunchKernelGGL((bias_gelu_vec_kernel<CT, 1>), grid, dim3(256), 0, s, C, ldc, M, N, bias, epi, tx);
  } else {
    const int64_t want = ((int64_t)M * N + 255) / 256;
    const int64_t cap = (int64_t)cu_count * 16;  // enough resident waves to saturate HBM
    const unsigned grid = (unsigned)(want < cap ? (want > 0 ? want : 1) : cap);
    hipLaunchKernelGGL((bias_gelu_scalar_kernel<CT>), dim3(grid), dim3(256), 0, s, C, ldc, M, N, bias, epi);
  }
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
