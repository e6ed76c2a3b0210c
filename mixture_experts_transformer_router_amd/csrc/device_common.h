// Device helpers shared by the gfx950 kernels: element loads/stores, the two
// expert activations and wave64 reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float -> bf16 bits, round to nearest even (NaN stays a quiet NaN); the
// conversion is gfx950's v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
// two floats -> packed bf16 pair (a in the low half)
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return static_cast<uint32_t>(f32_to_bf16(a)) | (static_cast<uint32_t>(f32_to_bf16(b)) << 16);
}

// fp64 -> nearest bf16, ties to even, with one rounding.  The fp32 rounding
// f of v is exact for the decision unless f lies exactly on a bf16 midpoint
// (low 16 bits 0x8000) while v does not: no midpoint can lie strictly between
// v and its nearest fp32.  In that case the sign of |v| - |f| decides.
// Finite values in bf16's normal range (NaN is kept as a quiet NaN).
__device__ __forceinline__ uint16_t f64_to_bf16(double v) {
  const float f = static_cast<float>(v);
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  if ((u & 0xffffu) == 0x8000u) {
    const double rest = fabs(v) - fabs(static_cast<double>(f));
    if (rest > 0.0) return static_cast<uint16_t>((u + 0x8000u) >> 16);  // magnitude up
    if (rest < 0.0) return static_cast<uint16_t>(u >> 16);              // magnitude down
  }
  return static_cast<uint16_t>((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

template <typename T> __device__ __forceinline__ float load_f32(const T* p, size_t i);
template <> __device__ __forceinline__ float load_f32<float>(const float* p, size_t i) { return p[i]; }
template <> __device__ __forceinline__ float load_f32<uint16_t>(const uint16_t* p, size_t i) {
  return bf16_to_f32(p[i]);
}

template <typename T> __device__ __forceinline__ void store_f32(T* p, size_t i, float v);
template <> __device__ __forceinline__ void store_f32<float>(float* p, size_t i, float v) { p[i] = v; }
template <> __device__ __forceinline__ void store_f32<uint16_t>(uint16_t* p, size_t i, float v) {
  p[i] = f32_to_bf16(v);
}

// Logistic function with the hardware exp2 and reciprocal (about 2 ulp).
__device__ __forceinline__ float sigmoidf_(float z) { return __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// v clipped to [lo, hi]; NaN stays NaN: IEEE 754-2019 maximum / minimum
// (gfx950 v_maximum3_f32 / v_minimum3_f32; the older min / max / median
// instructions return the other operand for a NaN input).
__device__ __forceinline__ float clip_nan(float v, float lo, float hi) {
  return __builtin_elementwise_minimum(__builtin_elementwise_maximum(v, lo), hi);
}

// Expert activation.  act 0: clipped SwiGLU (gate clipped to [0, limit], up to
// [-limit, limit], h = g' * sigmoid(alpha g') * u').  act 1: h = g sigmoid(g) u.
// A NaN gate or up value gives a NaN h.
__device__ __forceinline__ float expert_act(int act, float g, float u, float alpha, float limit) {
  if (act == 0) {
    const float gc = clip_nan(g, 0.f, limit);
    const float uc = clip_nan(u, -limit, limit);
    return gc * sigmoidf_(alpha * gc) * uc;
  }
  return g * sigmoidf_(g) * u;
}

// Wave64 reductions (all lanes receive the result).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
// Index of an empty arg-max candidate.
constexpr int kNoIndex = 0x7fffffff;

// (v1, i1) precedes (v2, i2) in the order (value descending, index
// ascending); an empty candidate (index kNoIndex) follows everything.  Values
// must not be NaN (callers map NaN to -inf), so the order is total.
__device__ __forceinline__ bool precedes(float v1, int i1, float v2, int i2) {
  if (i1 == kNoIndex) return false;
  if (i2 == kNoIndex) return true;
  return v1 > v2 || (v1 == v2 && i1 < i2);
}

// Arg-max over the wave in that order; every lane receives the same result.
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    float ov = __shfl_xor(v, o, 64);
    int oi = __shfl_xor(i, o, 64);
    if (precedes(ov, oi, v, i)) { v = ov; i = oi; }
  }
}

}  // namespace moe

namespace moe {

// ---- gfx950 MFMA operands -------------------------------------------------
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// D = A (16 x 32) * B (32 x 16) + C, bf16 inputs, fp32 accumulate.
// Lane l supplies A row (l % 16), k = 8 (l / 16) .. +7 and B column (l % 16),
// the same k; it receives D rows 4 (l / 16) .. +3 of column (l % 16).
__device__ __forceinline__ f32x4_t mfma_16x16x32(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8_t load_bf16x8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(p));
}
// Streaming (read-once) variant: non-temporal hint so weights do not evict
// reusable lines from the caches.
__device__ __forceinline__ bf16x8_t load_bf16x8_stream(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8_t, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p)));
}
__device__ __forceinline__ bf16x8_t zero_bf16x8() {
  return __builtin_bit_cast(bf16x8_t, u32x4_t{0u, 0u, 0u, 0u});
}

}  // namespace moe
