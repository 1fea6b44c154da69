// The static device scratch of tq_decode_attn_no_alloc: a file-scope device
// array, so that the call needs no allocation at all.  Each GPU the library
// runs on holds its own copy of the array from module load until the process
// ends.  In host code the array's name is only a stand-in for the symbol, so
// its device address is looked up once per device (with that device current)
// and that address, never the name, is what the kernels receive.
#include <mutex>

#include "tq_internal.h"

namespace tq {

namespace {
constexpr int kMaxDevices = 64;
__device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t no_alloc_scratch(void** out) {
  int dev = -1;
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
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace tq
