// Library-held scratch for the call that allocates nothing
// (sd_accept_reject_noalloc): one file-scope device array per GPU, whose
// device address is looked up once per device and kept.
//
// In host code `scratch` names a host-side stand-in, not device memory: the
// kernels must only ever see the address hipGetSymbolAddress returns for the
// current device, never the array's name.

#include <mutex>

#include "common.h"
#include "sd_verify.h"

namespace {

constexpr size_t kScratchBytes = SD_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

size_t sdv_noalloc_scratch_bytes() { return kScratchBytes; }

// Device address of the current device's scratch array (looked up on the
// first call per device, with that device current).
hipError_t sdv_noalloc_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
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
