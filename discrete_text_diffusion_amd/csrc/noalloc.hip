// Device scratch for the allocation-free Step entry point (dg_step_sample_noalloc): a fixed array in
// the library's code object, so every GPU that loads the library holds its own copy until the process
// ends.  Host code never names the array directly: it uses the address looked up here, once per
// device, with that device current.
#include <mutex>

#include "internal.h"

namespace dg {

static __device__ __align__(256) char scratch[STATIC_SCRATCH_BYTES];

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex g_mu;
void* g_scratch[MAX_DEVICES] = {};
}  // namespace

hipError_t static_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace dg
