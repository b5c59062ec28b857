// Scratch memory of the entry points that allocate nothing (fa_fwd_splitkv_noalloc): one
// file-scope device array, of which every GPU the library runs on holds its own copy until
// the process ends. Host code never uses the array's name as an address (on the host it
// names a stand-in, not device memory): the device address of each GPU's copy is looked up
// once per device with hipGetSymbolAddress, with that device current, and kept.
#include <hip/hip_runtime.h>

#include <mutex>

#include "fa_internal.h"

namespace fa {
namespace {

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices];  // device address of `scratch` on each device, once looked up

}  // namespace

hipError_t scratch_buffer(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
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

}  // namespace fa
