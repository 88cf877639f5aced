// Library-owned device scratch for the entry point that allocates nothing
// (draft_mask_and_perm_noalloc): a file-scope device array whose address is
// looked up once per device. In host code the array's name is only a
// host-side stand-in; every host use goes through the address that
// hipGetSymbolAddress returned for the current device.
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.h"

namespace lvsa {
namespace {

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices];  // per-device address of `scratch`, set on first use

}  // namespace

hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace lvsa
