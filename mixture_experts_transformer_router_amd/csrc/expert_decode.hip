// Expert stages for a few tokens (T <= 16): every expert holds at most 16
// sorted rows, so each stage is a stream over the active experts' weights.
//
//   gate|up:  h[r][f] = act(x[t] . Wg[e][f] + bg[e][f], x[t] . Wu[e][f] + bu[e][f])
//   down:     y[r][n] = h[r] . Wd[e][n] + bd[e][n]
//
// (MaxText GPT-OSS weight mapping "MOE EXPERTS"; glm4_moe_lite.go
// SwitchMLP.Forward and SharedExperts.Forward.)
//
// One block per (16 weight rows, expert); blocks of experts without rows exit
// at once.  The weight rows are the 16-row operand of
// v_mfma_f32_16x16x32_bf16 and the expert's tokens (zero-padded to 16) the
// 16-column operand, so no cross-lane reduction is needed inside a
// wavefront.  The block's 4 wavefronts split the reduction dimension into
// contiguous quarters; their partial tiles are added in wavefront order
// (deterministic).  Each lane reads 32 contiguous bytes of a weight row per
// step of 64 elements (the two halves feed two MFMAs whose k order is the
// same for both operands), so four lanes cover one 128-byte line.
#include "device_common.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kWaves = 4;
constexpr int kRows = 16;

struct DecodeArgs {
  const uint16_t* a;          // gate|up: x [T, lda]; down: h [rows, lda]
  int lda;
  const int32_t* row_token;   // gate|up: token of each sorted row; down: nullptr
  const uint16_t* w0;         // [E, N, K]: down, or gate
  const uint16_t* w1;         // up (gate|up only)
  const uint16_t* bias0;      // [E, N] or nullptr
  const uint16_t* bias1;
  const uint16_t* sh_w0;      // shared expert [N_sh, K_sh] or nullptr
  const uint16_t* sh_w1;
  int N, K, N_sh, K_sh;
  int E;
  const int32_t* offsets;     // [E_all + 1]
  uint16_t* out;
  int ldo;
  int act;
  float alpha, limit;
};

template <bool GATED>
__global__ __launch_bounds__(64 * kWaves) void decode_kernel(DecodeArgs a) {
  __shared__ float red[kWaves][GATED ? 2 : 1][kRows][kRows + 1];

  const int e = blockIdx.y;
  const bool shared = e >= a.E;
  const int N = shared ? a.N_sh : a.N;
  const int K = shared ? a.K_sh : a.K;
  const int n0 = blockIdx.x * kRows;
  if (n0 >= N) return;
  const int m0 = a.offsets[e];
  const int m = a.offsets[e + 1] - m0;  // <= 16 on this path
  if (m <= 0) return;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int row = lane & 15, kg = lane >> 4;

  // A operand: weight row n0 + row
  const bool row_ok = n0 + row < N;
  const size_t wrow = (size_t)(row_ok ? n0 + row : n0) * K;
  const uint16_t* W0 = (shared ? a.sh_w0 : a.w0 + (size_t)e * a.N * a.K) + wrow;
  const uint16_t* W1 = GATED ? (shared ? a.sh_w1 : a.w1 + (size_t)e * a.N * a.K) + wrow : nullptr;
  // B operand: token slot `row` of this expert
  const bool tok_ok = row < m;
  const int brow = tok_ok ? (a.row_token ? a.row_token[m0 + row] : m0 + row) : 0;
  const uint16_t* B = a.a + (size_t)brow * a.lda;

  f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  const int steps = (K + 63) / 64;
  const int s_begin = (steps * wv) / kWaves, s_end = (steps * (wv + 1)) / kWaves;
#pragma unroll 4
  for (int s = s_begin; s < s_end; ++s) {
    const int k = 64 * s + 16 * kg;
    const bool k0 = k < K, k1 = k + 8 < K;  // K % 8 == 0
    const bf16x8_t b0 = (tok_ok && k0) ? load_bf16x8(B + k) : zero_bf16x8();
    const bf16x8_t b1 = (tok_ok && k1) ? load_bf16x8(B + k + 8) : zero_bf16x8();
    const bf16x8_t g0 = (row_ok && k0) ? load_bf16x8_stream(W0 + k) : zero_bf16x8();
    const bf16x8_t g1 = (row_ok && k1) ? load_bf16x8_stream(W0 + k + 8) : zero_bf16x8();
    acc0 = mfma_16x16x32(g0, b0, acc0);
    acc0 = mfma_16x16x32(g1, b1, acc0);
    if constexpr (GATED) {
      const bf16x8_t u0 = (row_ok && k0) ? load_bf16x8_stream(W1 + k) : zero_bf16x8();
      const bf16x8_t u1 = (row_ok && k1) ? load_bf16x8_stream(W1 + k + 8) : zero_bf16x8();
      acc1 = mfma_16x16x32(u0, b0, acc1);
      acc1 = mfma_16x16x32(u1, b1, acc1);
    }
  }
  // D[weight row][token slot]: lane holds rows 4 kg + r of column `row`
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    red[wv][0][4 * kg + r][row] = acc0[r];
    if constexpr (GATED) red[wv][1][4 * kg + r][row] = acc1[r];
  }
  __syncthreads();
  // epilogue: thread -> (weight row, token slot), weight row fastest
  const int er = tid & 15, slot = tid >> 4;
  if (slot >= m || n0 + er >= N) return;
  float v0 = 0.f, v1 = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    v0 += red[w][0][er][slot];
    if constexpr (GATED) v1 += red[w][1][er][slot];
  }
  const int n = n0 + er;
  if (!shared && a.bias0) v0 += bf16_to_f32(a.bias0[(size_t)e * N + n]);
  if constexpr (GATED) {
    if (!shared && a.bias1) v1 += bf16_to_f32(a.bias1[(size_t)e * N + n]);
    v0 = expert_act(shared ? 1 : a.act, v0, v1, a.alpha, a.limit);
  }
  a.out[(size_t)(m0 + slot) * a.ldo + n] = f32_to_bf16(v0);
}

DecodeArgs base_args(const Layer& L, const Work& W) {
  DecodeArgs d{};
  d.E = L.E;
  d.offsets = W.offsets;
  d.act = L.act;
  d.alpha = L.alpha;
  d.limit = L.limit;
  return d;
}

}  // namespace

hipError_t launch_gate_up_decode(const Layer& L, const Work& W, hipStream_t s) {
  DecodeArgs d = base_args(L, W);
  d.a = static_cast<const uint16_t*>(L.x);
  d.lda = L.d;
  d.row_token = W.row_token;
  d.w0 = static_cast<const uint16_t*>(L.wg);
  d.w1 = static_cast<const uint16_t*>(L.wu);
  d.bias0 = static_cast<const uint16_t*>(L.bg);
  d.bias1 = static_cast<const uint16_t*>(L.bu);
  d.sh_w0 = static_cast<const uint16_t*>(L.sh_wg);
  d.sh_w1 = static_cast<const uint16_t*>(L.sh_wu);
  d.N = L.F; d.K = L.d; d.N_sh = L.F_sh; d.K_sh = L.d;
  d.out = static_cast<uint16_t*>(W.h);
  d.ldo = L.F_max();
  const dim3 grid((L.F_max() + kRows - 1) / kRows, L.n_experts_all());
  decode_kernel<true><<<grid, 64 * kWaves, 0, s>>>(d);
  return hipGetLastError();
}

hipError_t launch_down_decode(const Layer& L, const Work& W, hipStream_t s) {
  DecodeArgs d = base_args(L, W);
  d.a = static_cast<const uint16_t*>(W.h);
  d.lda = L.F_max();
  d.row_token = nullptr;
  d.w0 = static_cast<const uint16_t*>(L.wd);
  d.bias0 = static_cast<const uint16_t*>(L.bd);
  d.sh_w0 = static_cast<const uint16_t*>(L.sh_wd);
  d.N = L.d; d.K = L.F; d.N_sh = L.d; d.K_sh = L.F_sh;
  d.out = static_cast<uint16_t*>(W.y);
  d.ldo = L.d;
  const dim3 grid((L.d + kRows - 1) / kRows, L.n_experts_all());
  decode_kernel<false><<<grid, 64 * kWaves, 0, s>>>(d);
  return hipGetLastError();
}

}  // namespace moe
