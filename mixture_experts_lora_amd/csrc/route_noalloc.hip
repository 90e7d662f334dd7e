// moe_route_noalloc: moe_route without a caller workspace, for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid allocation).  The routing scratch (the
// per-block histogram and every pair's in-block rank) lives in a file-scope
// device array that each GPU holds until the process ends.  Every call on
// one GPU uses that GPU's copy, so calls that overlap on one GPU race.
#include <mutex>

#include "../../include/moe_lora.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr size_t NOALLOC_BYTES = MOE_ROUTE_NOALLOC_SCRATCH_BYTES;
static_assert(NOALLOC_BYTES % 256 == 0, "scratch size");

// Host code must not pass this name to a kernel: on the host it is only a
// stand-in for the symbol.  Its device address comes from scratch_ptr().
static __device__ __attribute__((aligned(256))) unsigned char scratch[NOALLOC_BYTES];

constexpr int MAX_DEV = 64;
std::mutex g_mu;
void* g_ptr[MAX_DEV];  // device address of `scratch` on each device, once looked up

// This device's copy of `scratch`: looked up on the first call with the
// device current, then kept.  Null if the device index is out of range or the
// lookup fails.
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEV) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_ptr[dev] = p;
  }
  return g_ptr[dev];
}

}  // namespace
}  // namespace moe

extern "C" moe_status moe_route_noalloc(const moe_dims* dm, const float* logits,
                                        const moe_routing* out, void* stream) {
  const size_t need = moe_route_workspace_bytes(dm);
  // invalid dims: moe_route reports which error before it touches the workspace
  if (need == 0) return moe_route(dm, logits, out, nullptr, 0, stream);
  if (need > moe::NOALLOC_BYTES) return MOE_ERROR_UNSUPPORTED;
  void* p = moe::scratch_ptr();
  if (!p) return MOE_ERROR_LAUNCH;
  // the routing kernels write every scratch element they read: nothing needs
  // clearing between calls
  return moe_route(dm, logits, out, p, moe::NOALLOC_BYTES, stream);
}
