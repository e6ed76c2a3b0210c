// Combine: back to token order with the routing weights.
//
//   out[t] = sum_{j = 0..k-1} w[t,j] * y[pos[t*k + j]]   (+ y[shared row of t])
//
// summed in fp32 in increasing j, the shared expert added last, then rounded
// once to the output type (glm4_moe_lite.go, MoE.Forward: weighted sum over
// the k expert outputs, then the shared experts added).  In a MoE block the
// block input x[t] is added after that, before the rounding (MoEBlock.Forward:
// the block returns its input plus the MoE output).  Deterministic: no
// atomics; each output element is produced by one thread.
#include "device_common.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

struct CombineArgs {
  const void* y;
  const float* w;
  const int32_t* pos;
  int T, d, k, shared;
  const void* resid;  // [T, d] rows added last, or nullptr
  void* out;
};

// VEC elements per thread (8 for bf16 = 16 bytes, 4 for fp32).
template <typename TE, int VEC>
__global__ __launch_bounds__(kThreads) void combine_kernel(CombineArgs a) {
  const int t = blockIdx.x;
  const TE* Y = static_cast<const TE*>(a.y);
  TE* O = static_cast<TE*>(a.out);
  const int P = a.T * a.k;
  __shared__ int rows[17];
  __shared__ float wts[16];
  if (threadIdx.x < a.k) {
    rows[threadIdx.x] = a.pos[(size_t)t * a.k + threadIdx.x];
    wts[threadIdx.x] = a.w[(size_t)t * a.k + threadIdx.x];
  }
  if (threadIdx.x == 0) rows[16] = P + t;
  __syncthreads();
  const int nvec = a.d / VEC;
  // block (t, c) covers vectors c kThreads .. c kThreads + kThreads - 1 of row t
  {
    const int v = blockIdx.y * kThreads + threadIdx.x;
    if (v >= nvec) return;
    float acc[VEC];
#pragma unroll
    for (int q = 0; q < VEC; ++q) acc[q] = 0.f;
    for (int j = 0; j < a.k; ++j) {
      const size_t base = (size_t)rows[j] * a.d + (size_t)v * VEC;
      const float wj = wts[j];
#pragma unroll
      for (int q = 0; q < VEC; ++q) acc[q] = fmaf(wj, load_f32(Y, base + q), acc[q]);
    }
    if (a.shared) {
      const size_t base = (size_t)rows[16] * a.d + (size_t)v * VEC;
#pragma unroll
      for (int q = 0; q < VEC; ++q) acc[q] += load_f32(Y, base + q);
    }
    const size_t ob = (size_t)t * a.d + (size_t)v * VEC;
    if (a.resid) {
      const TE* R = static_cast<const TE*>(a.resid);
#pragma unroll
      for (int q = 0; q < VEC; ++q) acc[q] += load_f32(R, ob + q);
    }
#pragma unroll
    for (int q = 0; q < VEC; ++q) store_f32(O, ob + q, acc[q]);
  }
}

}  // namespace

hipError_t launch_combine(const Layer& L, const Work& W, hipStream_t s) {
  CombineArgs a;
  a.y = W.y; a.w = W.w; a.pos = W.pos;
  a.T = L.T; a.d = L.d; a.k = L.k; a.shared = L.has_shared() ? 1 : 0;
  a.resid = L.x_resid;
  a.out = L.out;
  // one block per token and kThreads vectors of its row: a row of a few
  // thousand elements takes a few blocks, each thread one vector
  const int vec = L.dt == MOE_F32 ? 4 : 8;
  const dim3 grid(L.T, (L.d / vec + kThreads - 1) / kThreads);
  if (L.dt == MOE_F32) combine_kernel<float, 4><<<grid, kThreads, 0, s>>>(a);
  else combine_kernel<uint16_t, 8><<<grid, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace moe
