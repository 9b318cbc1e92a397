// Group-quantized weights: shared definitions of the quantized-matmul kernels (gfx950 only).
//
// C = epi(alpha * X W^T + beta * C [+ bias]) with w[j][k] = s[j][k / G] * q[j][k] + o[j][k / G],
// the quantized matmul of "X3: Metal GEMM", section 7 (decode: a matrix-vector product bound by
// the weight bytes; prefill: a matrix product), dequantisation fused into the multiply-add.
#pragma once

#include "common.hpp"

namespace tgemm {

struct QParams {
  const void* X;        // M x K activations (f16 / bf16), row stride ldx
  const uint8_t* W;     // N rows of codes, ldw bytes apart
  const void* S;        // scales, N rows of ldg values (activation type)
  const void* O;        // offsets, same layout
  void* C;              // M x N output, row stride ldc
  const float* bias;    // fp32[N] or null
  int64_t ldx, ldw, ldg, ldc;
  int M, N, K, bits, group;
  float alpha, beta;
  uint32_t epi;
};

// A 16-bit activation-type word to float.
template <int XT>
__device__ __forceinline__ float x16_to_float(uint32_t h) {
  if constexpr (XT == BF16) return bf16_bits_to_float(h);
  else return f16_bits_to_float(h);
}

template <int XT>
__device__ __forceinline__ float load_x16(const void* base, int64_t idx) {
  return x16_to_float<XT>(reinterpret_cast<const uint16_t*>(base)[idx]);
}

// Code k of weight row j: one byte, or a nibble (low nibble for even k).
__device__ __forceinline__ uint32_t q_code(const QParams& p, int64_t j, int64_t k) {
  const uint8_t* row = p.W + j * p.ldw;
  if (p.bits == 8) return row[k];
  return (row[k >> 1] >> (4 * (k & 1))) & 15u;
}

// The epilogue of one output: alpha * acc, beta * C_in, bias, GELU, rounded once on store.
template <int XT>
__device__ __forceinline__ void q_store(const QParams& p, int64_t m, int64_t j, float acc) {
  const int64_t idx = m * p.ldc + j;
  const float cin = p.beta != 0.0f ? load_as_float<XT>(p.C, idx) : 0.0f;
  const float bj = (p.epi & EPI_BIAS) ? p.bias[j] : 0.0f;
  store_from_float<XT>(p.C, idx, epilogue_value<XT>(acc, p.alpha, p.beta, cin, bj, p.epi));
}

}  // namespace tgemm
