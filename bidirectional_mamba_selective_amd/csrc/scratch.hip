// The library's fixed device scratch buffer, for the entry point that allocates nothing
// (bimamba_scan_fwd_noalloc): the chunked scan's workspace lives in one file-scope device array of
// kScratchBytes instead of caller memory.  Each GPU the library runs on holds its own copy of the
// array from the time the code object is loaded until the process ends.
//
// In host code the array's name is only a stand-in for the symbol, not a device address: its address
// on the current device comes from hipGetSymbolAddress, taken once per device and kept here.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "launch.h"

namespace bimamba {

namespace {

__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_addr[kMaxDevices];
std::mutex g_mu;

}  // namespace

hipError_t scratch_address(void** out) {
  *out = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_mu);
    p = g_addr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      // the device is current: the address is that device's copy of the array
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (p == nullptr) return hipErrorInvalidSymbol;
      g_addr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

}  // namespace bimamba
