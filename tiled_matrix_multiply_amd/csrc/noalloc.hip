// Static device scratch for gemm_run_noalloc, the entry point that allocates nothing (for
// callers that cannot call hipMalloc: code under graph capture, tight serving loops).
//
// `scratch` is a file-scope device array.  In host code its name is a host-side stand-in, not
// a device address: the handle takes the array's address on its device once, at gemm_create
// (hipGetSymbolAddress with that device current), and every launch uses that address.  Each
// device the library runs on holds its own copy of the array until the process ends.  It
// starts zeroed (device globals are zero-initialised when the code object loads); the one
// kernel that uses it (the K loop split across two workgroups) keeps tile t in slot t whatever
// the call's size and leaves each slot it used with its counter even and its flag at half the
// counter, which is the state the next call needs, so nothing has to be cleared per call.  Calls on one device share the array, so calls
// that overlap on one device (different streams, unsynchronised) race on it.
#include "common.hpp"

namespace tgemm {
// 128 workspace slots (each a tile's counter and flag, then its 256 x 128 fp32 partial sums):
// a 2048 x 2048 output, or any output of at most 128 such tiles.  16 MiB + 32 KiB.
constexpr int64_t kScratchBytes = 128 * kSplitSlotBytes;
}  // namespace tgemm

static __device__ __align__(256) uint8_t scratch[tgemm::kScratchBytes];

namespace tgemm {

// Device address of this device's copy of the scratch array (call with the device current).
hipError_t scratch_address(void** out) { return hipGetSymbolAddress(out, HIP_SYMBOL(scratch)); }

int64_t scratch_bytes() { return kScratchBytes; }

}  // namespace tgemm
