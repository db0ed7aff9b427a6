// The library's own prefill workspace, for the entry point that allocates
// nothing: one file-scope device array, which the loader reserves on every
// device the library's code is loaded on, for the life of the process.  On
// the host the array's name is only a stand-in for registration, never a
// device address; host code asks the runtime for each device's copy once
// (with that device current) and uses only the address it returns.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.hpp"

namespace qgemv {
namespace {

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_at[kMaxDevices] = {};

}  // namespace

hipError_t scratch_address(hipStream_t s, void** ptr) {
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  int dev = cur;
  if (s && (e = hipStreamGetDevice(s, &dev)) != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_at[dev]) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t back = hipSetDevice(cur);
      if (e == hipSuccess) e = back;
    }
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_at[dev] = p;
  }
  *ptr = g_at[dev];
  return hipSuccess;
}

}  // namespace qgemv
