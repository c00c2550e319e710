// moe_forward_noalloc: the whole layer with its workspace in a fixed device
// array of the library, for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc).  The kernels and their launch sequence are moe_forward's;
// only the workspace differs.
#include <hip/hip_runtime.h>

#include <atomic>

#include "api_internal.h"
#include "moe.h"

namespace {

// The workspace of every call on a device: one array per device, held from
// the library's first use on that device until the process ends.  In host
// code `scratch` names a host-side stand-in, not the device array; the
// device address comes from hipGetSymbolAddress (per device, below).
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch[kMaxDevices];

// Device address of the current device's array, looked up once per device
// with that device current.  Concurrent first calls look it up twice and
// store the same address.
int scratch_of_current_device(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
  void *p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return MOE_OK;
}

}  // namespace

extern "C" int moe_forward_noalloc(const moe_shape *s, const void *x, int act, const void *wg,
                                   const float *bias, const moe_expert_weights *w, void *y,
                                   int out, int32_t *topk_idx, float *topk_w, void *stream) {
  const size_t need = (s && w) ? moe_workspace_bytes(s, w->dtype) : 0;
  if (need == 0 || need > (size_t)MOE_NOALLOC_SCRATCH_BYTES)
    // Argument errors first; a valid call that needs more than the array
    // holds gets MOE_ERR_WORKSPACE.
    return moe::forward_impl(s, x, act, wg, bias, w, y, out, topk_idx, topk_w, nullptr, 0,
                             stream);
  void *ws = nullptr;
  const int st = scratch_of_current_device(&ws);
  if (st != MOE_OK) return st;
  return moe::forward_impl(s, x, act, wg, bias, w, y, out, topk_idx, topk_w, ws,
                           (size_t)MOE_NOALLOC_SCRATCH_BYTES, stream);
}
