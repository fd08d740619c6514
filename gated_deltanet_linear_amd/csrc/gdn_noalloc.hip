// gdn_noalloc.hip -- the library-owned device array that gdn_chunk_forward_noalloc uses as the
// chunked prefill's workspace, for callers that cannot allocate (the entry point itself is in
// gdn_abi.cpp).
//
// The workspace lives in `scratch`, a file-scope __device__ array of kNoallocScratchBytes. Each
// GPU the library runs on holds its own copy for the life of the process. In host code the name
// `scratch` is only a host-side stand-in, so the array's device address is looked up once per
// device with hipGetSymbolAddress (with that device current) and only that address is passed to
// the kernels. Every call on one GPU uses the same array: calls that overlap on one GPU (two
// streams, or two host threads) race on it. The kernels write every workspace byte they later
// read, so nothing needs clearing between calls.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/gdn.h"
#include "gdn_internal.h"

constexpr size_t kNoallocScratchBytes = (size_t)GDN_NOALLOC_SCRATCH_BYTES;

static __device__ __align__(256) char scratch[kNoallocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, or null

// Device address of the current device's scratch array (looked up on the first call per device).
hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

namespace gdn {

hipError_t noalloc_scratch(void** ptr, size_t* bytes) {
  *bytes = kNoallocScratchBytes;
  return scratch_address(ptr);
}

}  // namespace gdn
