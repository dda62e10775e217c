// moe_layer_forward_noalloc: the layer forward on a fixed scratch array that
// the library holds in device memory, for callers that cannot allocate (code
// under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc).  The work is moe_layer_forward's, unchanged; only the workspace
// comes from `scratch` instead of the caller.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/moe.h"
#include "kernels.hpp"

namespace {

// The scratch array: one copy per GPU, each at its own device address, held
// until the process ends.  In host code the name `scratch` is only a host-side
// stand-in; the device address comes from hipGetSymbolAddress (below).
__device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per
// device with that device current.  Returns hipSuccess and sets *p.
hipError_t scratch_ptr(void** p) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_ptr[dev]) {
    void* q = nullptr;
    e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!q) return hipErrorInvalidSymbol;
    g_ptr[dev] = q;
  }
  *p = g_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" int moe_layer_forward_noalloc(const void* x, const int32_t* token_ids,
                                         const void* w_router, const float* bias,
                                         const moe_expert_weights* routed,
                                         const moe_expert_weights* shared, int64_t T, int D,
                                         int E, int k, int I, int I_shared, moe_route mode,
                                         moe_dtype act, uint32_t flags, void* y, void* stream) {
  // The size check comes first and is host-only: a layer too large for the
  // scratch array is refused before any device call.
  if (T >= 0 && D > 0 && E > 0 && k > 0 && I > 0 && routed) {
    const size_t need = moe_layer_workspace_bytes(T, D, E, k, I, shared ? I_shared : 0, act,
                                                  routed->dtype);
    if (need > (size_t)MOE_NOALLOC_SCRATCH_BYTES)
      return moe::set_error(MOE_ERR_WORKSPACE,
                            "moe_layer_forward_noalloc: the layer needs %zu bytes of scratch, "
                            "above the fixed %zu (MOE_NOALLOC_SCRATCH_BYTES); use "
                            "moe_layer_forward with a workspace",
                            need, (size_t)MOE_NOALLOC_SCRATCH_BYTES);
  }
  void* ws = nullptr;
  const hipError_t e = scratch_ptr(&ws);
  if (e != hipSuccess)
    return moe::set_error(MOE_ERR_HIP, "moe_layer_forward_noalloc: scratch address: %s",
                          hipGetErrorString(e));
  return moe_layer_forward(x, token_ids, w_router, bias, routed, shared, T, D, E, k, I, I_shared,
                           mode, act, flags, y, ws, (size_t)MOE_NOALLOC_SCRATCH_BYTES, stream);
}
