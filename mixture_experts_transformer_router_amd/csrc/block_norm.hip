// RMSNorm in front of the MoE layer of a block (glm4_moe_lite.go,
// MoEBlock.Forward: the MoE input is PostAttentionLayerNorm(h), an RMSNorm
// with Config.RMSNormEps):
//
//   xn[t] = x[t] / sqrt(mean_i x[t,i]^2 + eps) * w
//
// xn is an array of the layer's element type and the router's choices depend
// on it, so it is computed in fp64 and rounded ONCE to bf16 (fp32), to
// nearest-even: the result is the correctly rounded value of the formula (the
// fp64 errors are ~2^-50 relative, far inside the half-ulp margins of bf16 or
// fp32).  One block per token row: the sum of squares in a fixed order
// (per-thread strided partial sums, a wave butterfly, then the 8 wave sums in
// order).  A thread keeps its ITER x VEC elements of the row in registers
// between the two passes (rows up to 4 x VEC x 512 elements); longer
// rows are read twice (ITER = 0).  fp64 costs nothing here: the kernel moves
// 2-4 bytes per ~5 flops.
#include "device_common.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 512;

template <typename TE> __device__ __forceinline__ void store_f64(TE* p, size_t i, double v);
template <> __device__ __forceinline__ void store_f64<float>(float* p, size_t i, double v) {
  p[i] = static_cast<float>(v);  // v_cvt_f32_f64: round to nearest even
}
template <> __device__ __forceinline__ void store_f64<uint16_t>(uint16_t* p, size_t i, double v) {
  p[i] = f64_to_bf16(v);
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

template <typename TE, int VEC, int ITER>
__global__ __launch_bounds__(kThreads) void rmsnorm_kernel(const TE* __restrict__ x, const TE* __restrict__ w,
                                                           float eps, int d, TE* __restrict__ xn) {
  const TE* xr = x + (size_t)blockIdx.x * d;
  TE* outr = xn + (size_t)blockIdx.x * d;
  constexpr int R = ITER > 0 ? ITER * VEC : 1;
  float keep[R];
  double ss = 0.0;
  if constexpr (ITER > 0) {
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      const int i = (it * kThreads + threadIdx.x) * VEC;
#pragma unroll
      for (int q = 0; q < VEC; ++q) {
        keep[it * VEC + q] = i < d ? load_f32(xr, i + q) : 0.f;
        const double v = keep[it * VEC + q];
        ss = fma(v, v, ss);
      }
    }
  } else {
    for (int i = threadIdx.x * VEC; i < d; i += kThreads * VEC) {
#pragma unroll
      for (int q = 0; q < VEC; ++q) {
        const double v = load_f32(xr, i + q);
        ss = fma(v, v, ss);
      }
    }
  }
  ss = wave_sum_f64(ss);
  __shared__ double part[kThreads / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  double tot = 0.0;
#pragma unroll
  for (int i = 0; i < kThreads / 64; ++i) tot += part[i];
  const double r = 1.0 / sqrt(tot / d + static_cast<double>(eps));
  if constexpr (ITER > 0) {
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      const int i = (it * kThreads + threadIdx.x) * VEC;
      if (i < d) {
#pragma unroll
        for (int q = 0; q < VEC; ++q)
          store_f64(outr, i + q, static_cast<double>(keep[it * VEC + q]) * r * static_cast<double>(load_f32(w, i + q)));
      }
    }
  } else {
    for (int i = threadIdx.x * VEC; i < d; i += kThreads * VEC) {
#pragma unroll
      for (int q = 0; q < VEC; ++q)
        store_f64(outr, i + q, static_cast<double>(load_f32(xr, i + q)) * r * static_cast<double>(load_f32(w, i + q)));
    }
  }
}

template <typename TE, int VEC>
hipError_t launch_t(const Layer& L, const Work& W, hipStream_t s) {
  const TE* x = static_cast<const TE*>(L.x);
  const TE* w = static_cast<const TE*>(L.norm_w);
  TE* xn = static_cast<TE*>(W.xn);
  const int iters = (L.d + kThreads * VEC - 1) / (kThreads * VEC);
  switch (iters) {
    case 1: rmsnorm_kernel<TE, VEC, 1><<<L.T, kThreads, 0, s>>>(x, w, L.eps, L.d, xn); break;
    case 2: rmsnorm_kernel<TE, VEC, 2><<<L.T, kThreads, 0, s>>>(x, w, L.eps, L.d, xn); break;
    case 3: rmsnorm_kernel<TE, VEC, 3><<<L.T, kThreads, 0, s>>>(x, w, L.eps, L.d, xn); break;
    case 4: rmsnorm_kernel<TE, VEC, 4><<<L.T, kThreads, 0, s>>>(x, w, L.eps, L.d, xn); break;
    default: rmsnorm_kernel<TE, VEC, 0><<<L.T, kThreads, 0, s>>>(x, w, L.eps, L.d, xn); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rmsnorm(const Layer& L, const Work& W, hipStream_t s) {
  // d % 8 == 0 (the library's limits), so VEC divides every row
  return L.dt == MOE_F32 ? launch_t<float, 4>(L, W, s) : launch_t<uint16_t, 8>(L, W, s);
}

}  // namespace moe
