// Fixed device scratch for moe_layer_forward_noalloc: the layer's workspace
// as a file-scope device array (one copy per GPU, held until the process
// ends), so that the call needs no allocation at all.
//
// Host code never passes `scratch` itself to a kernel: in host code that name
// is only a stand-in for the symbol. Its device address on the current GPU
// comes from hipGetSymbolAddress, looked up once per device (with that device
// current) and kept in a per-device table.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/moe.h"
#include "kernels.h"

namespace moe {

static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

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
    if (!p) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return hipSuccess;
}

}  // namespace moe
