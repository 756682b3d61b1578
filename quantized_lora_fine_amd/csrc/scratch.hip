// Device-resident workspace of the allocation-free forward (nf4lora_fwd_noalloc).
//
// Callers that cannot allocate (code under graph capture, tight serving
// loops, harnesses that forbid hipMalloc) still need the forward's scratch
// space: the padded adapter copies, the saved s*T and the split partials and
// counters of the adapter product.  This file holds it as one file-scope
// device array of kNoAllocScratchBytes per GPU, created with the code object
// and held until the process ends.
//
// On the host, `scratch` names a host-side stand-in, not the device memory:
// every device address of it comes from hipGetSymbolAddress, looked up once
// per device with that device current (each GPU holds its own copy at its
// own address) and kept in g_scratch.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.hpp"

static __device__ __align__(256) unsigned char scratch[nf4k::kNoAllocScratchBytes];

namespace nf4k {

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return hipSuccess;
}

}  // namespace nf4k
