// Device-resident decode workspace for callers that cannot allocate
// (kvq_decode_noalloc): the split partials live in a file-scope device array
// instead of caller memory. Each GPU the library runs on holds its own copy
// of the array, at its own address, until the process ends.
//
// In host code `scratch` names a host-side stand-in, not device memory: its
// device address is looked up once per device with hipGetSymbolAddress (with
// that device current) and only that address is ever handed to kernels.
#include <atomic>
#include <mutex>

#include "kvq_internal.h"

namespace {

__device__ __attribute__((aligned(256))) uint8_t scratch[kvq::kStaticWorkspaceBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
std::atomic<void*> g_addr[kMaxDevices];

}  // namespace

hipError_t kvq_static_workspace(hipStream_t stream, void** addr) {
  int dev = 0;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lk(g_mu);
    p = g_addr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      int cur = 0;
      e = hipGetDevice(&cur);
      if (e != hipSuccess) return e;
      if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      const hipError_t back = cur != dev ? hipSetDevice(cur) : hipSuccess;
      if (e != hipSuccess) return e;
      if (back != hipSuccess) return back;
      if (p == nullptr) return hipErrorInvalidSymbol;
      g_addr[dev].store(p, std::memory_order_release);
    }
  }
  *addr = p;
  return hipSuccess;
}
