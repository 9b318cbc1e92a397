// Measurement kernels (used by the benchmark; not part of the GEMM).
//
//  * clock_probe_kernel: the shader clock the chip is running at.  Each one-wave workgroup reads
//    the shader-clock cycle counter (s_memtime) and the constant-rate counter (s_memrealtime,
//    its rate is the device's wall-clock rate) at its start and again once a fixed span of the
//    constant clock has passed; cycles / ticks x the constant rate is the clock.  Queued right
//    behind a timed run of a kernel it reads the clock that run left the chip at (the power
//    controller moves the clock on millisecond scales, the probe lasts tens of microseconds).
//    The spin is bounded twice: by the constant clock and by an iteration cap, so every wave
//    ends whatever the counters do.
//  * bandwidth_probe_kernel: the practical HBM ceiling, the measured side of the roofline that
//    "Case Study: The Tiled GEMM" gets from its bandwidth script: a grid-stride stream of
//    16-byte loads (read only) or loads and stores (a copy), four in flight per thread.
#include "common.hpp"

namespace tgemm {

namespace {

typedef uint32_t u32x4p __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(64) void clock_probe_kernel(uint64_t* out, uint64_t ticks) {
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  uint64_t r = r0;
  for (int i = 0; i < (1 << 16) && r - r0 < ticks; ++i) r = __builtin_amdgcn_s_memrealtime();
  const uint64_t c1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) {
    uint64_t* o = out + 4 * (int64_t)blockIdx.x;
    o[0] = c0;
    o[1] = r0;
    o[2] = c1;
    o[3] = r1;
  }
}

constexpr int kBwThreads = 256;

template <bool COPY>
__global__ __launch_bounds__(kBwThreads) void bandwidth_probe_kernel(const u32x4p* __restrict__ src,
                                                                     u32x4p* __restrict__ dst,
                                                                     int64_t n, uint32_t* sink) {
  const int64_t stride = (int64_t)gridDim.x * kBwThreads;
  int64_t i = (int64_t)blockIdx.x * kBwThreads + threadIdx.x;
  u32x4p acc = u32x4p{0u, 0u, 0u, 0u};
  for (; i + 3 * stride < n; i += 4 * stride) {
    const u32x4p a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    if constexpr (COPY) {
      dst[i] = a;
      dst[i + stride] = b;
      dst[i + 2 * stride] = c;
      dst[i + 3 * stride] = d;
    } else {
      acc ^= a ^ b ^ c ^ d;
    }
  }
  for (; i < n; i += stride) {
    const u32x4p a = src[i];
    if constexpr (COPY) dst[i] = a;
    else acc ^= a;
  }
  if constexpr (!COPY) {
    // keeps the loads: the store happens only for one improbable checksum
    if ((acc[0] ^ acc[1] ^ acc[2] ^ acc[3]) == 0x9e3779b9u) sink[0] = acc[0];
  }
}

}  // namespace

hipError_t launch_clock_probe(uint64_t* out, int workgroups, uint64_t ticks, hipStream_t s) {
  hipLaunchKernelGGL(clock_probe_kernel, dim3(workgroups), dim3(64), 0, s, out, ticks);
  return hipGetLastError();
}

hipError_t launch_bandwidth_probe(const void* src, void* dst, int64_t bytes, uint32_t* sink,
                                  int cu_count, hipStream_t s) {
  const int64_t n = bytes / 16;
  const int64_t want = (n + kBwThreads - 1) / kBwThreads;
  const int64_t cap = (int64_t)cu_count * 8;
  const unsigned grid = (unsigned)(want < cap ? (want > 0 ? want : 1) : cap);
  const u32x4p* in = reinterpret_cast<const u32x4p*>(src);
  u32x4p* out = reinterpret_cast<u32x4p*>(dst);
  if (dst) hipLaunchKernelGGL(bandwidth_probe_kernel<true>, dim3(grid), dim3(kBwThreads), 0, s, in, out, n, sink);
  else hipLaunchKernelGGL(bandwidth_probe_kernel<false>, dim3(grid), dim3(kBwThreads), 0, s, in, out, n, sink);
  return hipGetLastError();
}

}  // namespace tgemm
