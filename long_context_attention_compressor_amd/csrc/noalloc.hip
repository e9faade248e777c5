// noalloc.hip -- the library's one fixed device scratch area, for the entry
// point that allocates nothing (indexer_topk_noalloc).
//
// `scratch` is a file-scope device array: every GPU the library runs on holds
// its own copy at its own address, from the first use until the process
// ends.  On the host the name `scratch` is only a stand-in for the symbol,
// never a device address: the address on each device is looked up once, with
// that device current, and only that address is handed to kernels.
#include <mutex>

#include "lac_internal.h"

namespace lac {

namespace {

__device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_addr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  *ptr = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_addr[dev] = p;
  }
  *ptr = g_addr[dev];
  return hipSuccess;
}

}  // namespace lac
