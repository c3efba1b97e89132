// Library-owned scratch for the forward entry point that allocates nothing
// (vlp_varlen_attn_fwd_noalloc): the device-built tile metadata that
// vlp_varlen_attn_fwd keeps in a caller-supplied workspace lives here instead,
// in one file-scope device array per GPU.
//
// In host code `scratch` is only a host-side stand-in for the symbol; the
// device address of each GPU's copy comes from hipGetSymbolAddress, taken
// once per device (with that device current) and kept.  Every launch gets
// that address, never the array's name.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "vlp_internal.h"

namespace vlp {
namespace {

__device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_addr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  *ptr = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_addr[dev] = p;
  }
  *ptr = g_addr[dev];
  return hipSuccess;
}

}  // namespace vlp
