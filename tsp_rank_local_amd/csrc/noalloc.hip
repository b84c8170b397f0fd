// Device scratch for the entry point that allocates nothing: one fixed-size
// array per GPU, resident from the library's load until the process ends.
//
// In host code the array's name stands for a host-side shadow, not for a
// device address, so it is never passed to a kernel or a copy. The device
// address is looked up once per device, with that device current, through
// hipGetSymbolAddress, and kept; every use goes through that address.
#include <mutex>

#include "tsp_internal.h"

namespace tsp {

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_addr[kMaxDevices];  // device address of `scratch` on each device, once looked up
}  // namespace

hipError_t noalloc_scratch(hipStream_t stream, void **addr) {
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  if (stream != nullptr) {
    hipDevice_t sdev = -1;
    e = hipStreamGetDevice(stream, &sdev);
    if (e != hipSuccess) return e;
    if ((int)sdev != cur) return hipErrorInvalidDevice;  // the lookup must run with the stream's device current
  }
  if (cur < 0 || cur >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_addr[cur] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_addr[cur] = p;
  }
  *addr = g_addr[cur];
  return hipSuccess;
}

}  // namespace tsp
