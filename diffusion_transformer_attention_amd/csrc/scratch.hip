// Static device scratch for the one entry point that must not allocate
// (dit_attn_fwd_balanced_noalloc): callers under HIP graph capture, in tight
// serving loops, or in harnesses that forbid hipMalloc.
//
// The array lives in this file's code object, so every GPU the library runs
// on holds its own copy (DIT_SCRATCH_BYTES) until the process ends.  In host
// code the name `scratch` is only a host-side stand-in for the symbol: its
// device address is looked up here once per device, with that device
// current, and the kernels receive that address as an ordinary pointer.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/dit_attn.h"
#include "launch.h"

static __device__ __align__(256) unsigned char scratch[DIT_SCRATCH_BYTES];

namespace ditattn {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch` on each device, once looked up

}  // namespace

hipError_t scratch_buffer(void** out, size_t* bytes) {
  *out = nullptr;
  *bytes = 0;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  *bytes = DIT_SCRATCH_BYTES;
  return hipSuccess;
}

}  // namespace ditattn
