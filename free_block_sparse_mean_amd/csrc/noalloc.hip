// Library-owned scratch for the entry point that allocates nothing
// (sol_attn_fwd_noalloc): one static device array per GPU, holding the
// pre-pass workspace of one call. The array lives in the code object's device
// memory from the moment the library is loaded on a device until the process
// ends; nothing is allocated or freed per call.
//
// In host code `scratch` names a host-side stand-in, not a device address:
// the device address is looked up once per device with hipGetSymbolAddress
// (with that device current) and only that address is handed to kernels.
#include <mutex>
#include <vector>

#include "sol_internal.hpp"

namespace sol {
namespace {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mutex;
std::vector<void*> g_scratch_ptr;   // per device id; null until looked up

}  // namespace

hipError_t noalloc_scratch(void** out) {
  *out = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if ((size_t)dev >= g_scratch_ptr.size()) g_scratch_ptr.resize(dev + 1, nullptr);
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

}  // namespace sol
