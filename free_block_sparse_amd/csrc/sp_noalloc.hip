// Fixed device scratch for the allocation-free entry point
// (sparsepr_attention_noalloc): one file-scope array per GPU, held until the
// process ends.  Host code never passes the array's name to a kernel: the
// name is a host-side stand-in, not a device address.  Its address on each
// device is looked up once, with that device current, and kept per device.
#include <map>
#include <mutex>

#include "sp_kernels.h"

namespace sp {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

// Device address of this device's scratch array (the current device).
hipError_t noalloc_scratch(void** ptr) {
  static std::mutex mu;
  static std::map<int, void*> addr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(mu);
  auto it = addr.find(dev);
  if (it == addr.end()) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    it = addr.emplace(dev, p).first;
  }
  *ptr = it->second;
  return hipSuccess;
}

}  // namespace sp
