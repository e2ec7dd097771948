// Fixed device scratch for the entry points that allocate nothing.
//
// One file-scope array per device, kScratchBytes long, held until the process
// ends.  Host code never passes the array's name to a kernel (on the host that
// name is a stand-in, not a device address): the device address is taken once
// per device with hipGetSymbolAddress, with that device current, and kept.
#include <hip/hip_runtime.h>

#include <mutex>

#include "cq_internal.h"

namespace {

static __device__ __align__(256) unsigned char scratch[cqi::kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_addr[kMaxDevices] = {};

}  // namespace

namespace cqi {

hipError_t scratch_address(void** out) {
  *out = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_addr[dev] = p;
  }
  *out = g_addr[dev];
  return hipSuccess;
}

}  // namespace cqi
