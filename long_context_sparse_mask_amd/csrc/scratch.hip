// Library-owned scratch memory for the entry point that allocates nothing
// (hip_sparse_attn_noalloc): a file-scope device array, one per GPU, held by
// the process until it ends.
//
// In host code the array's name is only a stand-in for the symbol, not a
// device address.  Its address on a GPU comes from hipGetSymbolAddress, called
// once per device with that device current; every use from the host (kernel
// arguments) goes through that address, never through the name.
#include <hip/hip_runtime.h>

#include <mutex>

#include "hipsa_internal.h"

static_assert(hipsa::kNoAllocScratchBytes == HIPSA_NOALLOC_SCRATCH_BYTES,
              "the scratch size must match the header");

namespace {

__device__ __align__(256) unsigned char scratch[hipsa::kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_ptr[kMaxDevices];  // scratch address on each device, once looked up

}  // namespace

namespace hipsa {

// The scratch array's address on the device that runs `stream` (the current
// device for the null stream).  The first call for a device looks it up with
// that device current and restores the caller's current device afterwards.
hipError_t noalloc_scratch(hipStream_t stream, void **ptr) {
  int dev = 0;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    int cur = 0;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    const hipError_t e2 = cur != dev ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess) return e;
    if (e2 != hipSuccess) return e2;
    if (!p) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return hipSuccess;
}

}  // namespace hipsa
