// noalloc.hip -- the scratch memory of the allocation-free decode step
// (lca_decode_step_noalloc): one file-scope device array per GPU, whose
// address is resolved once per device and kept.  In host code the array's
// name is only a stand-in for the symbol; kernels receive the resolved
// device address.
#include <mutex>

#include "lca_internal.h"

namespace lca {

static __device__ __align__(256) uint8_t scratch[NOALLOC_SCRATCH_BYTES];

constexpr int NOALLOC_MAX_DEVICES = 64;
static void* g_scratch[NOALLOC_MAX_DEVICES];
static std::mutex g_scratch_mu;

hipError_t noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= NOALLOC_MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));       // with `dev` current
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return hipSuccess;
}

}  // namespace lca
