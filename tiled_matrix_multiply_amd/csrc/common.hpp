// Shared device-side definitions of the tiled GEMM library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tgemm {

enum DType : int { F32 = 0, F16 = 1, BF16 = 2, E4M3 = 3 };
enum : uint32_t { EPI_BIAS = 1u, EPI_GELU = 2u };

// Arguments every GEMM kernel receives (by value, in the kernel-argument segment).
struct GemmParams {
  const void* A;
  const void* B;
  void* C;
  const float* bias;
  int64_t lda, ldb, ldc;  // leading dimensions in elements
  int M, N, K;
  int tiles_m, tiles_n;   // workgroup tiles along M and N
  float alpha;            // alpha * scale_a * scale_b
  float beta;
  uint32_t epi;           // EPI_BIAS | EPI_GELU
};

template <int DT> struct DTypeInfo;
template <> struct DTypeInfo<F32> { static constexpr int bytes = 4; };
template <> struct DTypeInfo<F16> { static constexpr int bytes = 2; };
template <> struct DTypeInfo<BF16> { static constexpr int bytes = 2; };
template <> struct DTypeInfo<E4M3> { static constexpr int bytes = 1; };

// ------------------------------------------------------------------ element conversions --

__device__ __forceinline__ float bf16_bits_to_float(uint32_t h) {
  return __uint_as_float(h << 16);
}

__device__ __forceinline__ float f16_bits_to_float(uint32_t h) {
  _Float16 v = __builtin_bit_cast(_Float16, (uint16_t)h);
  return (float)v;
}

// OCP E4M3 byte -> float, exact: exponent bias 7, subnormals m * 2^-9, NaN at S.1111.111.
__device__ __forceinline__ float e4m3_bits_to_float(uint32_t q) {
  const uint32_t s = (q >> 7) & 1u, e = (q >> 3) & 15u, m = q & 7u;
  float v;
  if (e == 0) v = (float)m * 0x1p-9f;
  else if (e == 15 && m == 7) v = __builtin_nanf("");
  else v = __uint_as_float(((e + 120u) << 23) | (m << 20));  // (1 + m/8) * 2^(e-7)
  return s ? -v : v;
}

// float -> storage (round to nearest even), returned in the low bits.
__device__ __forceinline__ uint32_t float_to_bf16_bits(float v) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v);
}
__device__ __forceinline__ uint32_t float_to_f16_bits(float v) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v);
}

template <int DT>
__device__ __forceinline__ float load_as_float(const void* base, int64_t idx) {
  if constexpr (DT == F32) return reinterpret_cast<const float*>(base)[idx];
  else if constexpr (DT == F16) return f16_bits_to_float(reinterpret_cast<const uint16_t*>(base)[idx]);
  else if constexpr (DT == BF16) return bf16_bits_to_float(reinterpret_cast<const uint16_t*>(base)[idx]);
  else return e4m3_bits_to_float(reinterpret_cast<const uint8_t*>(base)[idx]);
}

template <int CT>
__device__ __forceinline__ void store_from_float(void* base, int64_t idx, float v) {
  if constexpr (CT == F32) reinterpret_cast<float*>(base)[idx] = v;
  else if constexpr (CT == F16) reinterpret_cast<uint16_t*>(base)[idx] = (uint16_t)float_to_f16_bits(v);
  else reinterpret_cast<uint16_t*>(base)[idx] = (uint16_t)float_to_bf16_bits(v);
}

// ------------------------------------------------------------------------------ epilogue --

// GELU in its exact form x * Phi(x) = 0.5 x (1 + erf(x / sqrt 2)), in fp32, written with the
// complementary error function, 0.5 x erfc(-x / sqrt 2): the same function without the
// cancellation of 1 + erf(.) for negative x.
__device__ __forceinline__ float gelu_erf(float x) {
  return 0.5f * x * erfcf(x * -0.70710678118654752f);
}

// GELU for 16-bit outputs: x * Phi(x) with erfc from the rational approximation of
// Abramowitz & Stegun, Handbook of Mathematical Functions, formula 7.1.26 (absolute error at
// most 1.5e-7 for erf): erfc(y) ~ t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) exp(-y^2),
// t = 1 / (1 + p y), y >= 0.  Branch free: one reciprocal, one exp2, five FMAs.  In fp32 the
// result is within 1.1e-7 (1 + |x|) of x Phi(x), about 2% of a bf16 unit in the last place.
__device__ __forceinline__ float gelu_as7126(float x) {
  const float y = fabsf(x) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, y, 1.0f));
  float poly = fmaf(1.061405429f, t, -1.453152027f);
  poly = fmaf(poly, t, 1.421413741f);
  poly = fmaf(poly, t, -0.284496736f);
  poly = fmaf(poly, t, 0.254829592f);
  const float e = poly * t * __builtin_amdgcn_exp2f(-(y * y) * 1.4426950408889634f);  // erfc(y)
  const float phi = x >= 0.0f ? fmaf(-0.5f, e, 1.0f) : 0.5f * e;
  return x * phi;
}

// GELU at the precision the output type can hold: the device erfc for fp32 outputs, the
// branch-free approximation above for fp16 / bf16 outputs.
template <int CT>
__device__ __forceinline__ float gelu_out(float x) {
  if constexpr (CT == F32) return gelu_erf(x);
  else return gelu_as7126(x);
}

// alpha*acc (+ beta*c_in) (+ bias) then GELU: the fused epilogue applied in registers.
template <int CT>
__device__ __forceinline__ float epilogue_value(float acc, float alpha, float beta, float c_in,
                                                float bias_j, uint32_t epi) {
  float v = alpha * acc;
  if (beta != 0.0f) v = fmaf(beta, c_in, v);
  if (epi & EPI_BIAS) v += bias_j;
  if (epi & EPI_GELU) v = gelu_out<CT>(v);
  return v;
}

}  // namespace tgemm
