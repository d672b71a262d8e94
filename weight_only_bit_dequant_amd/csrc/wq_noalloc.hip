// Device-resident scratch for the allocation-free entry point
// (wq_fp8_static_linear_noalloc): a file-scope device array of fixed size,
// one copy per GPU, alive until the process ends.  Host code never passes the
// array's name to a kernel (on the host it names a stand-in, not device
// memory): the first call on a device, with that device current, resolves
// the device address with hipGetSymbolAddress and keeps it per device.
#include <hip/hip_runtime.h>

#include <mutex>

#include "wq_internal.hpp"

namespace wq {

namespace {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return hipSuccess;
}

}  // namespace wq
