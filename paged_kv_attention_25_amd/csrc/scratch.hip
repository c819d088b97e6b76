// Static device scratch for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops, harnesses that forbid allocation): the
// decode's split partials live in a file-scope array instead of a caller workspace.
//
// The array's name is a host-side stand-in, not a device address. Its address on a
// device is looked up once per device (hipGetSymbolAddress, with that device current)
// and kept; only that address is ever handed to kernels. Each device holds its own
// copy until the process ends, and every call on a device shares it: calls that
// overlap on one device race on its contents.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "pka_kernels.h"

namespace pka {

namespace {

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_lookup;

}  // namespace

hipError_t static_scratch(hipStream_t stream, void** ptr) {
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  if (stream != nullptr) {
    // The kernels run on the stream's device; the scratch must be that device's copy.
    hipDevice_t sdev = -1;
    err = hipStreamGetDevice(stream, &sdev);
    if (err != hipSuccess) return err;
    if (sdev != dev) return hipErrorInvalidDevice;
  }
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_lookup);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (err != hipSuccess) return err;
      if (p == nullptr) return hipErrorInvalidSymbol;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

}  // namespace pka
