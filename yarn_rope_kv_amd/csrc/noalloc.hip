// Device scratch for the entry point that allocates nothing
// (yrk_decode_attention_noalloc): the split partials of decode attention
// live in one file-scope device array instead of a caller-provided
// workspace.  Each GPU the library runs on holds its own copy of the array
// until the process ends.
//
// In host code `scratch` names a host-side stand-in, not device memory: its
// device address is looked up once per device (hipGetSymbolAddress, with
// that device current) and only that address is ever handed to a kernel.
#include <mutex>

#include <hip/hip_runtime.h>

#include "yrk_internal.h"

namespace yrk {
namespace {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch[kMaxDevices];   // device address of `scratch`, per device ordinal

}  // namespace

hipError_t device_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mutex);
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

}  // namespace yrk
