// Library handle shared by the host-side entry points (internal; not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm.h"

struct gemm_handle {
  uint32_t magic;
  int device;
  int cu_count;
  int wall_clock_khz;  // rate of the constant-rate counter (s_memrealtime)
  void* scratch;       // this device's copy of the library's static scratch array (device address)
  int64_t scratch_bytes;
  char arch[64];
};

namespace tgemm {

constexpr uint32_t kHandleMagic = 0x47454d4du;  // "GEMM"

// Makes `dev` the current device for the scope of a launch and restores the caller's.
struct DeviceGuard {
  int prev = -1;
  bool switched = false;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) == hipSuccess && prev != dev && hipSetDevice(dev) == hipSuccess)
      switched = true;
  }
  ~DeviceGuard() {
    if (switched) (void)hipSetDevice(prev);
  }
};

}  // namespace tgemm
