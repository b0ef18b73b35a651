// Fixed scratch for svg_layer_forward_noalloc: callers that cannot allocate
// (code under graph capture, tight serving loops) get the layer's workspace
// from a file-scope device array instead of hipMalloc.
//
// Each GPU that loads the library holds its own copy of the array until the
// process ends.  In host code the array's name is only a stand-in for the
// symbol; its device address is taken once per device with
// hipGetSymbolAddress (with that device current) and kept, and only that
// address is ever handed to kernels or copies.
#include <mutex>

#include "svg_internal.h"

namespace svg {

static __device__ __attribute__((aligned(256))) unsigned char scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices] = {};
std::mutex g_scratch_mu;
}  // namespace

hipError_t static_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace svg
