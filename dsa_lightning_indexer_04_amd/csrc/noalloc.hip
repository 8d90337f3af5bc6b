// noalloc.hip -- the fixed device scratch of dsa_indexer_topk_noalloc.
//
// One file-scope device array per GPU, sized for the Top-K workspace of
// modest calls (a decode batch of 64 rows against 131072 keys needs 32.5
// MiB; the streaming route needs (4*topk + 640) * 8 bytes per row).  Host
// code never uses the array's name as an address: its address on the
// current device comes from hipGetSymbolAddress, once per device, and is
// cached here.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "kernels.h"

namespace dsa {

static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_addr[kMaxDevices] = {};
}  // namespace

int noalloc_scratch(void** ptr, std::string* err) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *err = std::string("hipGetDevice: ") + hipGetErrorString(e);
    return 1;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    *err = "device ordinal out of range";
    return 1;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      *err = std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e);
      return 1;
    }
    g_addr[dev] = p;
  }
  *ptr = g_addr[dev];
  return 0;
}

}  // namespace dsa
