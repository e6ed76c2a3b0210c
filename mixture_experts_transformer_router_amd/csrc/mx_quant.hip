// MXFP8 conversion of bf16 rows (OCP Microscaling Formats v1.0: E4M3
// elements with one e8m0 scale per 32 consecutive elements; the MXFP8 mode
// of glm4_moe_lite.go quantizationParams: groups of 32, 8 bits).  This is
// the activation side of the scaled-MFMA expert GEMMs: the token rows before
// gate|up and the hidden activation h before down.
//
// Per block of 32 values v (bf16, so exact in fp32):
//   s = floor(log2(max |v|)) - 8, clamped to [-127, 127]   (8: E4M3's largest exponent)
//   scale byte = s + 127; code_i = E4M3(v_i / 2^s), nearest-even, saturating at +-448.
// An all-zero block gets scale byte 0; a block with a NaN or an infinity gets
// the NaN scale 255 and zero codes.  v_i / 2^s is exact (a power-of-two
// scaling that cannot overflow, and that underflows only far below the
// smallest E4M3 step), so the codes are a pure function of the bf16 input.
#include "device_common.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kQuantThreads = 256;

// E4M3 code of a finite float, nearest-even, |v| >= 448 -> 448; the sign bit is v's.
__device__ __forceinline__ uint32_t e4m3_rne_sat(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  uint32_t code;
  if (a >= 0x43E00000u) {                 // 448 = 1.75 * 2^8, the largest normal
    code = 0x7Eu;
  } else if (a < 0x3C800000u) {           // below 2^-6: subnormal steps of 2^-9, codes 0..8
    code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.f);
  } else {                                // keep 3 mantissa bits, ties to even; rebias 127 -> 7
    const uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
    code = (r >> 20) - (120u << 3);
  }
  return sign | code;
}

// One thread per 32-element block of a row; blocks at or past K (row padding
// up to ldq) get zero codes and scale byte 0.
__global__ __launch_bounds__(kQuantThreads) void mx_quant_kernel(const uint16_t* __restrict__ src, int lds, int R,
                                                                 int K, uint8_t* __restrict__ q,
                                                                 uint8_t* __restrict__ sc, int ldq) {
  const int nb = ldq / 32;
  const long long i = (long long)blockIdx.x * kQuantThreads + threadIdx.x;
  if (i >= (long long)R * nb) return;
  const int row = (int)(i / nb), b = (int)(i % nb);
  uint4* dst = reinterpret_cast<uint4*>(q + (size_t)row * ldq + 32 * b);
  if (32 * b >= K) {
    dst[0] = make_uint4(0u, 0u, 0u, 0u);
    dst[1] = make_uint4(0u, 0u, 0u, 0u);
    sc[(size_t)row * nb + b] = 0;
    return;
  }
  const uint4* p = reinterpret_cast<const uint4*>(src + (size_t)row * lds + 32 * b);
  uint32_t w[16];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const uint4 x = p[c];
    w[4 * c] = x.x; w[4 * c + 1] = x.y; w[4 * c + 2] = x.z; w[4 * c + 3] = x.w;
  }
  // largest magnitude as fp32 bits (integer order = magnitude order; NaN and
  // infinity compare above every finite value)
  uint32_t amax = 0;
#pragma unroll
  for (int c = 0; c < 16; ++c) amax = max(amax, max((w[c] << 16) & 0x7fff0000u, w[c] & 0x7fff0000u));
  uint32_t out[8];
  uint32_t scale_byte;
  if (amax >= 0x7f800000u) {
    scale_byte = 255u;
#pragma unroll
    for (int c = 0; c < 8; ++c) out[c] = 0u;
  } else {
    // floor(log2 amax): the exponent field, or for an fp32 subnormal (bf16
    // subnormals are) the position of the top mantissa bit; amax = 0 gives
    // -150, clamped like every s below -127
    const int e = amax >= 0x00800000u ? (int)(amax >> 23) - 127 : (31 - __clz((int)amax)) - 149;
    const int s = max(e - 8, -127);        // e <= 127, so s <= 119
    scale_byte = (uint32_t)(s + 127);
    const float inv = __uint_as_float((uint32_t)(127 - s) << 23);  // 2^-s, 127 - s in [8, 254]
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const uint32_t lo = w[2 * c], hi = w[2 * c + 1];
      const uint32_t c0 = e4m3_rne_sat(__uint_as_float(lo << 16) * inv);
      const uint32_t c1 = e4m3_rne_sat(__uint_as_float(lo & 0xffff0000u) * inv);
      const uint32_t c2 = e4m3_rne_sat(__uint_as_float(hi << 16) * inv);
      const uint32_t c3 = e4m3_rne_sat(__uint_as_float(hi & 0xffff0000u) * inv);
      out[c] = c0 | (c1 << 8) | (c2 << 16) | (c3 << 24);
    }
  }
  dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
  dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
  sc[(size_t)row * nb + b] = (uint8_t)scale_byte;
}

}  // namespace

hipError_t launch_mx_quant(const void* src, int lds, int R, int K, uint8_t* q, uint8_t* sc, int ldq, hipStream_t s) {
  const long long n = (long long)R * (ldq / 32);
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)((n + kQuantThreads - 1) / kQuantThreads));
  mx_quant_kernel<<<grid, kQuantThreads, 0, s>>>(static_cast<const uint16_t*>(src), lds, R, K, q, sc, ldq);
  return hipGetLastError();
}

}  // namespace moe
