// The library's own device workspace for moba_attn_fwd_static: a fixed array
// in device memory (one copy per GPU, created when the code object is loaded
// on that GPU and held until the process ends), for callers that cannot
// allocate device memory.  Host code never uses the array's name as an
// address: on the host it names a stand-in, not the device copy.  The device
// address is looked up once per device with hipGetSymbolAddress, with that
// device current, and kept.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/moba.h"
#include "launch.h"

static __device__ __align__(256) unsigned char scratch[MOBA_STATIC_WORKSPACE_BYTES];

namespace moba {

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_static_mu;
void* g_static_ptr[kMaxDevices] = {};

}  // namespace

hipError_t static_workspace(void** ptr, size_t* bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_static_mu);
  if (!g_static_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr || (uintptr_t)p % 256 != 0) return hipErrorInvalidSymbol;
    g_static_ptr[dev] = p;
  }
  *ptr = g_static_ptr[dev];
  *bytes = MOBA_STATIC_WORKSPACE_BYTES;
  return hipSuccess;
}

}  // namespace moba
