// scratch.hip — the fixed device scratch behind pa_decode_attention_noalloc: a file-scope device
// array that holds the split-K partials of callers that cannot allocate device memory.  Each GPU
// the library runs on has its own copy of the array (at its own address), kept until the process
// ends; its device address is looked up once per device with hipGetSymbolAddress, and only that
// address is handed to kernels or copies (the array's name in host code is a host-side stand-in).
#include <hip/hip_runtime.h>

#include <atomic>

#include "pa_kernels.h"

namespace pa {
namespace {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDev = 64;
std::atomic<void *> g_scratch[kMaxDev];

}  // namespace

hipError_t noalloc_scratch(void **ptr) {
  *ptr = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDev) return hipErrorInvalidDevice;
  void *p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    // once per device, with that device current (two threads racing here store the same address)
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return hipSuccess;
}

}  // namespace pa
