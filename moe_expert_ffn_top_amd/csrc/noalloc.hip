// Library-owned scratch for the entry point that allocates nothing
// (moe_expert_ffn_mx_noalloc): the MX activation workspace (the MXFP8 codes
// and scales of x and h, or their bf16 values on the weight-streaming path)
// lives in one file-scope device array instead of a caller buffer.
//
// In host code `scratch` names a host-side stand-in, not the device array:
// passing it to a kernel would compile and then fault on the GPU.  The
// device address is looked up once per device, with that device current,
// through hipGetSymbolAddress, and only that address is handed to kernels.
// Each GPU holds its own copy of the array, at its own address, until the
// process ends; every call on a GPU shares that GPU's copy.
#include <hip/hip_runtime.h>

#include <mutex>

#include "moe_common.hpp"

namespace moe {

static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];
}  // namespace

hipError_t noalloc_scratch(void** out) {
  *out = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace moe
