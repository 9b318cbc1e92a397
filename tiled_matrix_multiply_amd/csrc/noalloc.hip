// Static device scratch for gemm_run_noalloc, the entry point that allocates nothing (for
// callers that cannot call hipMalloc: code under graph capture, tight serving loops).
//
// `scratch` is a file-scope device array.  In host code its name is a host-side stand-in, not
// a device address: the handle takes the array's address on its device once, at gemm_create
// (hipGetSymbolAddress with that device current), and every launch uses that address.  Each
// device the library runs on holds its own copy of the array until the process ends.  It
// starts zeroed (device globals are zero-initialised when the code object loads); the one
// kernel that uses it (the K loop split across two workgroups) leaves its per-tile counters
// even and its flags at half the counters after every call, which is the state the next call
// needs, so nothing has to be cleared per call.  Calls on one device share the array, so calls
// that overlap on one device (different streams, unsynchronised) race on it.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tgemm {
// 4 KiB of per-tile counters and flags (up to 512 tiles) and 128 tiles of 256 x 128 fp32
// partial sums: a 2048 x 2048 output, or any output of at most 128 such tiles.
constexpr int64_t kScratchBytes = (int64_t(16) << 20) + 4096;
}  // namespace tgemm

static __device__ __align__(256) uint8_t scratch[tgemm::kScratchBytes];

namespace tgemm {

// Device address of this device's copy of the scratch array (call with the device current).
hipError_t scratch_address(void** out) { return hipGetSymbolAddress(out, HIP_SYMBOL(scratch)); }

int64_t scratch_bytes() { return kScratchBytes; }

}  // namespace tgemm
