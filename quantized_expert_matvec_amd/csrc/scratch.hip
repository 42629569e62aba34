// scratch.hip -- the library's one piece of static device memory: the workspace
// of fmoe_moe_layer_noalloc, for callers that cannot allocate device memory.
//
// `scratch` is a file-scope device array; every GPU the library runs on holds its
// own copy, at its own address, until the process ends. In host code the name
// `scratch` is only a host-side stand-in, never a device address: the device
// address is looked up once per device with hipGetSymbolAddress (with that device
// current) and cached, and only that address is handed to kernels. Every call on
// one GPU shares that GPU's copy, so calls that overlap on one GPU race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "layout.h"

namespace fmoe {

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_ptr[kMaxDevices] = {};
}  // namespace

// The device address of the current device's `scratch` (looked up on the first
// call per device); hipSuccess and *out set, or the runtime's error.
hipError_t scratch_device_ptr(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace fmoe
