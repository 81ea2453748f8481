// Device-resident workspace for gdr_prefill_noalloc: callers that cannot allocate (code under HIP
// graph capture, tight serving loops) get the prefill's workspace from a fixed array in device
// memory instead of from their own allocation.
//
// The array is a file-scope __device__ variable: every GPU the library runs on holds its own copy,
// at its own address, from the first use of the library's code on that GPU until the process ends.
// Host code never passes the array's name to a kernel (on the host the name is only a stand-in):
// the first call on a device looks its address up with hipGetSymbolAddress, with that device
// current, and keeps it per device.
#include <hip/hip_runtime.h>

#include <mutex>

#include "gdr_internal.h"

namespace gdr {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(void** out) {
  *out = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace gdr
