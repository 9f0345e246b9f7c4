// Static device scratch for the entry point that allocates nothing
// (sink_window_attention_noalloc): the attention kernels' partial results of
// split query tiles and the fp8 quantiser's maxima, in one file-scope device
// array instead of memory allocated at kv_cache_create.  Every GPU the library
// runs on holds its own copy of the array, at its own address, until the
// process ends; host code must use that address (looked up here with
// hipGetSymbolAddress, once per device), never the array's name.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "launch.h"

namespace kvc {
namespace {

constexpr size_t kScratchBytes = kStaticScratchBytes;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_addr[kMaxDevices] = {};

}  // namespace

int static_scratch(void** ptr, size_t* bytes) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return -1;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_addr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return -1;
    }
    g_addr[dev] = p;
  }
  *ptr = g_addr[dev];
  if (bytes) *bytes = kScratchBytes;
  return 0;
}

}  // namespace kvc
