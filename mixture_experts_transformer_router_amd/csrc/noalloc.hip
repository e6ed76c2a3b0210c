// moe_ffn_forward_noalloc: the GPT-OSS-style layer without a workspace
// argument, for callers that cannot allocate device memory (work recorded
// under HIP graph capture, serving loops that forbid allocation).  The
// workspace is `scratch`, a fixed array in the library's device code: the
// loader gives every GPU the library runs on its own copy, held until the
// process ends.  Host code reaches a GPU's copy only through the address
// hipGetSymbolAddress returns with that GPU current (the array's name in host
// code is a host-side stand-in, not a device address).
#include <hip/hip_runtime.h>

#include <mutex>

#include "moe_internal.h"

namespace moe {
namespace {

__device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of `dev`'s copy of the scratch array, looked up once per
// device with that device current.
hipError_t scratch_of(int dev, void** out) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_scratch[dev]) {
    *out = g_scratch[dev];
    return hipSuccess;
  }
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
  void* p = nullptr;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (cur != dev) {
    const hipError_t e2 = hipSetDevice(cur);
    if (e == hipSuccess) e = e2;
  }
  if (e != hipSuccess) return e;
  if (reinterpret_cast<uintptr_t>(p) % 256) return hipErrorInvalidValue;
  g_scratch[dev] = p;
  *out = p;
  return hipSuccess;
}

}  // namespace
}  // namespace moe

extern "C" moe_status moe_ffn_forward_noalloc(const void* x, const void* router_w, const void* router_b,
                                               const void* w_gate, const void* b_gate, const void* w_up,
                                               const void* b_up, const void* w_down, const void* b_down, int T,
                                               int d, int d_ff, int E, int k, float alpha, float limit, void* out,
                                               moe_dtype dt, moe_routing_out* routing, hipStream_t stream) {
  moe::clear_error();
  // sizes first: a call that needs more than the scratch array launches nothing
  const size_t need = moe_ffn_workspace_bytes(T < 0 ? 0 : T, d, d_ff, E, k, dt, 0, 0);
  if (need != (size_t)-1 && need > (size_t)MOE_NOALLOC_SCRATCH_BYTES)
    return moe::set_error(MOE_ERR_WORKSPACE, "the layer needs more workspace than the scratch array holds "
                                             "(MOE_NOALLOC_SCRATCH_BYTES); use moe_ffn_forward");
  moe::Layer L;
  L.x = x; L.router_w = router_w; L.router_b = router_b;
  L.wg = w_gate; L.bg = b_gate; L.wu = w_up; L.bu = b_up; L.wd = w_down; L.bd = b_down;
  L.T = T; L.d = d; L.F = d_ff; L.E = E; L.k = k;
  L.act = MOE_ACT_CLIPPED_SWIGLU; L.alpha = alpha; L.limit = limit;
  L.dt = dt; L.wfmt = dt == MOE_F32 ? moe::WF_F32 : moe::WF_BF16;
  L.out = out;
  if (routing) L.routing = *routing;
  if (need == (size_t)-1 || T <= 0) return moe::run_layer(L, nullptr, 0, stream);  // argument errors, T == 0
  int dev = 0;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return moe::set_error(MOE_ERR_HIP, "cannot find the stream's device");
  if (dev < 0 || dev >= moe::kMaxDevices) return moe::set_error(MOE_ERR_UNSUPPORTED, "device ordinal >= 64");
  void* ws = nullptr;
  if ((e = moe::scratch_of(dev, &ws)) != hipSuccess)
    return moe::set_error(MOE_ERR_HIP, "hipGetSymbolAddress of the scratch array failed");
  return moe::run_layer(L, ws, MOE_NOALLOC_SCRATCH_BYTES, stream);
}
