// Static per-device scratch of clef_head_forward_noalloc, the entry point for
// callers that cannot allocate device memory.  The array lives in the device
// code object: every GPU the library runs on holds its own copy, at its own
// address, until the process ends.  In host code `scratch` only names a host
// stand-in for the symbol, so its device address is looked up once per device
// (with that device current) and only that address is ever handed to kernels
// or copies.
#include <hip/hip_runtime.h>

#include <mutex>
#include <vector>

#include "kernels.hpp"

static __device__ __align__(256) unsigned char scratch[clef::kNoallocScratchBytes];

namespace clef {

hipError_t noalloc_scratch(int device, void** out) {
  static std::mutex mu;
  static std::vector<void*> addr;   // device address of `scratch`, per device
  std::lock_guard<std::mutex> lk(mu);
  if ((int)addr.size() <= device) addr.resize(device + 1, nullptr);
  if (addr[device] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[device] = p;
  }
  *out = addr[device];
  return hipSuccess;
}

}  // namespace clef
