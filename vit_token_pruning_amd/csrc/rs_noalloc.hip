// Device-resident scratch for the entry points that allocate nothing (callers that cannot
// call hipMalloc: work under HIP graph capture, tight serving loops, harnesses that forbid
// allocation).  The array lives in the library's code object; the HIP runtime places one
// copy on every device the library runs on when the module is loaded there, and it stays
// until the process ends.  Host code must never pass the array's name to a kernel (in host
// code it is only a stand-in, not a device address): its device address is looked up
// once per device with hipGetSymbolAddress and that pointer is used everywhere.
#include <hip/hip_runtime.h>

#include <mutex>

#include "rs_launch.hpp"

namespace rs {
namespace {

static __device__ __align__(256) char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));   // the current device's copy
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace rs
