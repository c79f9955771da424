// noalloc.hip -- the static device scratch behind gla_fwd_framecausal_noalloc.
//
// Callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc) get a frame-causal
// forward whose workspace is this file-scope array instead of a buffer they
// pass in. Every GPU the library runs on holds its own copy of the array for
// the life of the process.
//
// In host code `scratch` names a host-side stand-in, not device memory: its
// device address on the current GPU comes from hipGetSymbolAddress, taken once
// per device on first use and kept here, and only that address is ever handed
// to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/gla.h"

namespace gla {
namespace {

static __device__ __align__(256) char scratch[GLA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_ptr[kMaxDevices] = {};

}  // namespace

// Device address of the current GPU's scratch array (set up on the first call
// on that device, with it current). Returns NULL and sets *err on failure.
void *noalloc_scratch(hipError_t *err) {
  int dev = -1;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void *p = nullptr;
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*err != hipSuccess) return nullptr;
    g_ptr[dev] = p;
  }
  return g_ptr[dev];
}

}  // namespace gla
