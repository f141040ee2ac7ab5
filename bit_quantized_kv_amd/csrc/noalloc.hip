// The library's fixed device scratch for callers that cannot allocate: a
// file-scope device array (one copy per GPU, held until the process ends)
// that tq_decode_attention_noalloc uses for its split-K partials instead of a
// caller workspace.  Its device address is looked up once per device and
// kept; host code never uses the array's name as an address.
#include <hip/hip_runtime.h>

#include <mutex>

#include "tq_internal.h"

namespace tq {

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(void **ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return hipSuccess;
}

}  // namespace tq
