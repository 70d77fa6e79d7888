// Library-owned slab workspace for conv_wgrad_noalloc (callers that cannot
// allocate device memory).
//
// `scratch` is a file-scope device array: every GPU the library runs on holds
// its own copy (kNoallocScratchBytes, zero-initialised when the code object is
// loaded) until the process ends.  In host code its name is only a stand-in
// for the device copy, so host code never passes it to a kernel or a copy: the
// device address is looked up once per device with hipGetSymbolAddress, with
// that device current, and that address is what the kernels receive.
//
// The slabs need no clearing (every stage-1 workgroup writes its whole slab
// tile before the fold reads it), so nothing here is zeroed per call.  Every
// call on one GPU shares that GPU's array and leaves the last call's partial
// sums in it: calls that overlap in time on one GPU (different streams, or
// different host threads) race on it.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "kernels.h"

namespace cw {

namespace {

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    if (!p || (reinterpret_cast<uintptr_t>(p) & 255u) != 0) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace cw
