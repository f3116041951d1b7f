// Scratch memory of the no-allocation attention entry point
// (up_prefill_attn_noalloc): a file-scope device array that every GPU the
// library runs on holds until the process ends, used instead of a
// caller-allocated workspace.
//
// In host code `scratch` names a host-side stand-in, not device memory;
// its device address on each GPU comes from hipGetSymbolAddress, taken
// once per device with that device current and kept per device, and only
// that address is ever passed to kernels.
#include <mutex>

#include "common.h"

namespace up {

__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  *ptr = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace up
