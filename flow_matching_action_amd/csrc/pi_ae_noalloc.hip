// The fixed device array behind pi_ae_sample_noalloc: the working memory of
// one call of the denoise loop for callers that cannot allocate (code under
// stream capture, tight serving loops).  Every GPU the library runs on holds
// its own copy of the array until the process ends; calls that overlap on one
// GPU share it and race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "pi_ae_kernels.h"

namespace pi_ae {

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    // the device address of this GPU's copy of the array (the array's name is
    // a host-side stand-in that no host code may pass to a kernel)
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace pi_ae
