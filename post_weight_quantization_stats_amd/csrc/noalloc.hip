// Library-owned scratch for the entry point that allocates nothing
// (awq_decode_gemm_tiled_noalloc): a file-scope device array, one copy per
// GPU, alive until the process ends.
//
// Host code must never use the array's name as a device address (on the host
// it names a host-side stand-in).  The device address of each GPU's copy is
// looked up once per device with hipGetSymbolAddress, with that device
// current, and cached; callers get only that address.
#include <mutex>

#include "awq_internal.h"

namespace awq {

namespace {

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_addr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  *ptr = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_addr[dev] = p;
  }
  *ptr = g_addr[dev];
  return hipSuccess;
}

}  // namespace awq
