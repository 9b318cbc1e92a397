// Shared device-side definitions of the tiled GEMM library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tgemm {

// E2M1 is OCP fp4: two elements per byte along the storage row, the even element in the
// low nibble.
enum DType : int { F32 = 0, F16 = 1, BF16 = 2, E4M3 = 3, E5M2 = 4, E2M1 = 5, E2M3 = 6, E3M2 = 7 };
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
  uint32_t epi;           // EPI_BIAS | EPI_GELU (kernel-private flags in the upper bits)
  // OCP microscaling (MX): E8M0 scale of row i of op(A) and k-block kb (32 elements of K) at
  // sa[i * ldsa + kb], of column j of op(B) at sb[j * ldsb + kb]; kblocks = K / 32.  Null for
  // per-tensor scaling (folded into alpha).
  const uint8_t* sa;
  const uint8_t* sb;
  int64_t ldsa, ldsb;
  int kblocks;
  // Group-quantized B (the matrix-core kernel with dequantisation): B holds codes, ldb bytes
  // per row of op(B)^T; code k of row j is worth qs[j*ldg + k/group] * q + qo[j*ldg + k/group]
  // (16-bit, the activation type).  Null otherwise.
  const void* qs;
  const void* qo;
  int64_t ldg;
  int group;
  // K loop split across workgroups: the workspace (null otherwise).  Two workgroups per tile:
  // one kSplitSlotBytes slot per output tile (below).  Stream-K: two kStreamSlotBytes slots
  // per workgroup of the device's largest grid (one per compute unit), then from byte
  // sk_cnt_off an [arrive, done] pair of 32-bit counters per output tile; sk_grid workgroups.
  uint8_t* sk_ws;
  int64_t sk_cnt_off;
  int sk_grid;
};

// Workspace slot of one 256 x 128 output tile of the K loop split across two workgroups: its
// [counter, flag] pair of 32-bit words in the first 256 bytes, then the first workgroup's fp32
// partial sums (256 x 128 floats).  Slot t serves tile t whatever the size of the call, so calls
// of different sizes can share a workspace without one call's partial sums landing on another
// tile's counter and flag.
constexpr int64_t kSplitSlotBytes = 256 + 256 * 128 * 4;

// Stream-K workspace slot: one 256 x 256 tile's fp32 partial sums.
constexpr int64_t kStreamSlotBytes = 256 * 256 * 4;

template <int DT> struct DTypeInfo;
template <> struct DTypeInfo<F32> { static constexpr int bytes = 4; };
template <> struct DTypeInfo<F16> { static constexpr int bytes = 2; };
template <> struct DTypeInfo<BF16> { static constexpr int bytes = 2; };
template <> struct DTypeInfo<E4M3> { static constexpr int bytes = 1; };
template <> struct DTypeInfo<E5M2> { static constexpr int bytes = 1; };
// The matrix-core kernels see packed fp4 rows as bytes (two elements each), and packed 6-bit
// rows as bytes too (four elements per three).
template <> struct DTypeInfo<E2M1> { static constexpr int bytes = 1; };
template <> struct DTypeInfo<E2M3> { static constexpr int bytes = 1; };
template <> struct DTypeInfo<E3M2> { static constexpr int bytes = 1; };

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

// OCP E5M2 byte -> float, exact: exponent bias 15, subnormals m * 2^-16, exponent 31 is
// infinity (m = 0) or NaN.
__device__ __forceinline__ float e5m2_bits_to_float(uint32_t q) {
  const uint32_t s = (q >> 7) & 1u, e = (q >> 2) & 31u, m = q & 3u;
  float v;
  if (e == 0) v = (float)m * 0x1p-16f;
  else if (e == 31) v = m ? __builtin_nanf("") : __builtin_inff();
  else v = __uint_as_float(((e + 112u) << 23) | (m << 21));  // (1 + m/4) * 2^(e-15)
  return s ? -v : v;
}

// OCP E2M1 4-bit code -> float, exact: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.
__device__ __forceinline__ float e2m1_bits_to_float(uint32_t q) {
  const uint32_t s = (q >> 3) & 1u, e = (q >> 1) & 3u, m = q & 1u;
  const float v = e == 0 ? 0.5f * (float)m : __uint_as_float(((e + 126u) << 23) | (m << 22));
  return s ? -v : v;
}

// OCP 6-bit floats (MX v1.0), no infinities or NaN, exact in fp32:
//   E2M3: 1 sign, 2 exponent (bias 1), 3 mantissa bits, subnormals m * 2^-3;
//   E3M2: 1 sign, 3 exponent (bias 3), 2 mantissa bits, subnormals m * 2^-4.
__device__ __forceinline__ float e2m3_bits_to_float(uint32_t q) {
  const uint32_t s = (q >> 5) & 1u, e = (q >> 3) & 3u, m = q & 7u;
  const float v = e == 0 ? 0.125f * (float)m : __uint_as_float(((e + 126u) << 23) | (m << 20));
  return s ? -v : v;
}
__device__ __forceinline__ float e3m2_bits_to_float(uint32_t q) {
  const uint32_t s = (q >> 5) & 1u, e = (q >> 2) & 7u, m = q & 3u;
  const float v = e == 0 ? 0.0625f * (float)m : __uint_as_float(((e + 124u) << 23) | (m << 21));
  return s ? -v : v;
}

// Element idx of packed 6-bit storage: bits 6 idx .. 6 idx + 5 of the little-endian byte
// string; the following byte is read only when the element reaches into it (an element never
// crosses its group of three bytes).
__device__ __forceinline__ uint32_t fp6_code(const void* base, int64_t idx) {
  const uint8_t* b = reinterpret_cast<const uint8_t*>(base);
  const int64_t bit = 6 * idx, by = bit >> 3;
  const uint32_t sh = (uint32_t)(bit & 7);
  uint32_t v = (uint32_t)b[by] >> sh;
  if (sh > 2u) v |= (uint32_t)b[by + 1] << (8u - sh);
  return v & 63u;
}

// OCP E8M0 block scale 2^(e - 127) (e = 255 is NaN), exact in fp32: 2^-126 and up are
// normal numbers (exponent field e), 2^-127 is the subnormal 0x00400000.
__device__ __forceinline__ float e8m0_to_float(uint32_t e) {
  if (e == 255u) return __builtin_nanf("");
  return e == 0u ? 0x1p-127f : __uint_as_float(e << 23);
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
  else if constexpr (DT == E4M3) return e4m3_bits_to_float(reinterpret_cast<const uint8_t*>(base)[idx]);
  else if constexpr (DT == E5M2) return e5m2_bits_to_float(reinterpret_cast<const uint8_t*>(base)[idx]);
  else if constexpr (DT == E2M3) return e2m3_bits_to_float(fp6_code(base, idx));
  else if constexpr (DT == E3M2) return e3m2_bits_to_float(fp6_code(base, idx));
  else return e2m1_bits_to_float((reinterpret_cast<const uint8_t*>(base)[idx >> 1] >> (4 * (idx & 1))) & 15u);
}

template <int CT>
__device__ __forceinline__ void store_from_float(void* base, int64_t idx, float v) {
  if constexpr (CT == F32) reinterpret_cast<float*>(base)[idx] = v;
  else if constexpr (CT == F16) reinterpret_cast<uint16_t*>(base)[idx] = (uint16_t)float_to_f16_bits(v);
  else reinterpret_cast<uint16_t*>(base)[idx] = (uint16_t)float_to_bf16_bits(v);
}

// Four consecutive outputs, rounded to nearest even, written to LDS at dst (16-byte aligned for
// fp32, 8-byte for 16-bit types).
template <int CT>
__device__ __forceinline__ void stage4(uint8_t* dst, const float* v) {
  typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
  if constexpr (CT == F32) {
    *reinterpret_cast<float4*>(dst) = float4{v[0], v[1], v[2], v[3]};
  } else if constexpr (CT == BF16) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t lo = __builtin_convertvector((f32x2_t{v[0], v[1]}), bf16x2_t);
    const bf16x2_t hi = __builtin_convertvector((f32x2_t{v[2], v[3]}), bf16x2_t);
    *reinterpret_cast<u32x2_t*>(dst) = u32x2_t{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
  } else {
    uint32_t h[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) h[e] = float_to_f16_bits(v[e]);
    *reinterpret_cast<u32x2_t*>(dst) = u32x2_t{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
  }
}


// ------------------------------------------------------------------------------ epilogue --

// GELU in its exact form x * Phi(x) = 0.5 x (1 + erf(x / sqrt 2)), in fp32, written with the
// complementary error function, 0.5 x erfc(-x / sqrt 2): the same function without the
// cancellation of 1 + erf(.) for negative x.
__device__ __forceinline__ float gelu_erf(float x) {
  return 0.5f * x * erfcf(x * -0.70710678118654752f);
}

// GELU for 16-bit outputs, x Phi(x) with a complementary error function that keeps a bounded
// relative error over the whole line, so that the negative tail, where x Phi(x) is tiny, is as
// accurate as the rest.  Hastings' form (the one of Abramowitz & Stegun 7.1.26), refitted for
// relative error (erfc_fit.py beside this file regenerates the constants):
//   erfc(z) = t P(t) exp(-z^2),  t = 1 / (1 + p z),  z >= 0,
// P of degree 7 fitted minimax in relative terms to exp(z^2) erfc(z) / t (6.5e-7), p = 0.46.
// The function takes y = x / 2, which the GEMM epilogue produces directly by halving alpha,
// beta and the bias (exact: a power-of-two scaling).  With w = |y| and z = |x| / sqrt 2 = sqrt 2 w,
//   x Phi(x) = (x + |x|) / 2 - |x| erfc(z) / 2 = (y + |y|) - w erfc(sqrt 2 w),
// which is x - x erfc(x / sqrt 2) / 2 for x >= 0 and x erfc(-x / sqrt 2) / 2 for x < 0, with no
// branch on the sign.  exp(-z^2) is 2^a with a = -2 log2(e) w^2 + 32: the extra 2^32 keeps the
// hardware exponential's result a normal number until x Phi(x) is below the fp32 range, and
// 2^-32 is folded into P's coefficients.  In fp32 (an emulation of this operation order over
// x in [-14.5, 14.5]) the result is within 1.9e-6 relative of x Phi(x) for x in [-6, 3] and
// within 1e-5 wherever x Phi(x) is a normal fp32 number; the far tail's error is the rounding
// of a.  That is under 1/390 of a bf16 and 1/48 of an fp16 unit roundoff.  w is clamped at 15
// (x at 30): exp(-z^2) is 0 there, so +inf maps to +inf; NaN propagates through y + |y|.
__device__ __forceinline__ float gelu16_half(float y) {
  constexpr float kp = (float)(0.46 * 1.41421356237309505);  // p sqrt 2
  constexpr float ka = (float)(-2.0 * 1.44269504088896341);  // -2 log2(e)
  constexpr float g0 = 2.5952709021e-01f * 0x1p-32f, g1 = 2.5955513782e-01f * 0x1p-32f;
  constexpr float g2 = 2.3121260461e-01f * 0x1p-32f, g3 = 1.8668765607e-01f * 0x1p-32f;
  constexpr float g4 = 5.3007917024e-02f * 0x1p-32f, g5 = 1.6868148381e-01f * 0x1p-32f;
  constexpr float g6 = -2.2630292169e-01f * 0x1p-32f, g7 = 6.7631682811e-02f * 0x1p-32f;
  const float w = fminf(fabsf(y), 15.0f);
  const float t = __builtin_amdgcn_rcpf(fmaf(w, kp, 1.0f));
  float h = fmaf(g7, t, g6);
  h = fmaf(h, t, g5);
  h = fmaf(h, t, g4);
  h = fmaf(h, t, g3);
  h = fmaf(h, t, g2);
  h = fmaf(h, t, g1);
  h = fmaf(h, t, g0);
  const float e = __builtin_amdgcn_exp2f(fmaf(w * w, ka, 32.0f));  // 2^32 exp(-z^2)
  return fmaf(-w, (t * h) * e, y + fabsf(y));
}

// The same GELU from x itself.
__device__ __forceinline__ float gelu16(float x) { return gelu16_half(0.5f * x); }

// GELU at the precision the output type can hold: the device erfc for fp32 outputs, the
// branch-free form above for fp16 / bf16 outputs.
template <int CT>
__device__ __forceinline__ float gelu_out(float x) {
  if constexpr (CT == F32) return gelu_erf(x);
  else return gelu16(x);
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
