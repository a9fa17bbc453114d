// The static scratch of the allocation-free prefill (gka_fwd_chunked_static): the segment
// workspace held in a device array of the library, GKA_STATIC_SCRATCH_BYTES per GPU.
#include <hip/hip_runtime.h>

#include <atomic>

#include "gka.h"
#include "gka_internal.hpp"

namespace {

// The per-segment (dH, dU) summaries, start states, gate products and norms of a multi-segment
// plan. Every word a call reads here is written earlier in the same call (summaries, then the
// scan in place), so nothing needs clearing between calls.
static __device__ __align__(256) unsigned char scratch[GKA_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device

}  // namespace

namespace gka {

hipError_t static_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    // concurrent first calls on one device store the same address
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return hipSuccess;
}

}  // namespace gka
