// The library's own device workspace, for callers that cannot allocate device memory.
//
// A file-scope device array (one copy per GPU, held from the code object's load until
// the process ends) stands in for the caller's workspace in splitkv_attn_scratch. In
// host code the array's name is not a device address: the address of each GPU's copy
// is looked up once per device with hipGetSymbolAddress, with that device current,
// and only that address is ever handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.hpp"

namespace splitkv {
namespace {

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace splitkv
