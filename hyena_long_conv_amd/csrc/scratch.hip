// scratch.hip -- the library's one static device buffer, the four-step
// intermediate of hyena_forward_static (for callers that cannot allocate).
//
// `scratch` is a file-scope device array: every GPU the library runs on
// holds its own copy, at its own address, from the module's load until the
// process ends.  Host code never uses the array's name as an address (on the
// host it only stands for the symbol); it asks the runtime for the device
// address once per device, with that device current, and keeps it.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "launch.hpp"

namespace hyena {

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;
}  // namespace

hipError_t static_scratch(void** ptr, int64_t* bytes) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!p) return hipErrorInvalidSymbol;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  *bytes = kStaticScratchBytes;
  return hipSuccess;
}

}  // namespace hyena
