// The scratch array of moe_forward_noalloc: a file-scope device array that
// serves as that entry point's workspace, so that the call allocates no
// device memory (for callers that cannot: code under graph capture, tight
// serving loops, harnesses that forbid hipMalloc).  Each device that loads
// the library holds its own copy, at its own address, until the process
// ends.  In host code `scratch` names a host-side stand-in, not a device
// address, so host code uses only the address hipGetSymbolAddress returns.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/moe.h"
#include "internal.h"

namespace {

__device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices];     // device address of `scratch`, per device, once looked up

}  // namespace

namespace moe {

hipError_t noalloc_scratch(int dev, void** ptr) {
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return hipSuccess;
}

}  // namespace moe
