// Decode without a caller workspace: the partial results of the split KV axis live in a
// file-scope device array, one per GPU, sized kNoAllocScratchBytes, for callers that cannot
// allocate (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc). Its device address comes from hipGetSymbolAddress, once per device with that
// device current; the array's name itself is a host-side stand-in and never reaches a kernel.
#include "launch.h"

#include <atomic>
#include <mutex>

namespace attn {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

static std::atomic<void*> g_scratch_ptr[kMaxDevices];
static std::mutex g_scratch_mu;

hipError_t noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

}  // namespace attn
