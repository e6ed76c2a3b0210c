// The bf16 router block (MFMA logits for 16 tokens, then the expert choice)
// as a device function of the block's index, so that the router's launch and
// a launch that also carries other work run the same code.  Included by
// route.hip and expert_gemm_mfma.hip (device code of one translation unit
// each).
#pragma once

#include "route_common.h"

namespace moe {
namespace {

// ---- bf16: MFMA logits -----------------------------------------------------
constexpr int kMfmaTokens = 16;
#ifndef MOE_ROUTE_UNROLL
#define MOE_ROUTE_UNROLL 4
#endif
#ifndef MOE_ROUTE_TREE
#define MOE_ROUTE_TREE 1
#endif

// EG = groups of 16 experts (E <= 16 * EG).  WAVES split the input dimension.
// Their partial tiles are added either in wavefront order (sequential) or,
// with TREE, pairwise in a fixed tree (wave w += wave w + n/2 for n = WAVES,
// WAVES/2, ..., 2), both independent of timing.
template <int EG, int WAVES, bool TREE, bool NORM>
__device__ __forceinline__ void route_mfma_block(const RouteArgs& a, int blk) {
  constexpr int EP = 16 * EG;
  constexpr int kMfmaWaves = WAVES;
  __shared__ float lg[kMfmaTokens][EP + 1];
  __shared__ float part[TREE ? WAVES / 2 : 1][TREE ? EG * 4 * 64 : 1];
  __shared__ int cnt[EP];
  __shared__ double ssq[NORM ? WAVES : 1][kMfmaTokens];
  const uint16_t* x = static_cast<const uint16_t*>(a.x);
  const uint16_t* wr = static_cast<const uint16_t*>(a.wr);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int t0 = blk * kMfmaTokens;
  const int E = a.E, d = a.d;
  for (int e = tid; e < EP; e += 64 * kMfmaWaves) cnt[e] = 0;

  const int tok = t0 + (lane & 15);
  const int kg = lane >> 4;
  const bool tok_ok = tok < a.T;
  const uint16_t* xr = x + (size_t)(tok_ok ? tok : 0) * d;
  f32x4_t acc[EG];
#pragma unroll
  for (int g = 0; g < EG; ++g) acc[g] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // Batches of B steps: all loads of a batch are issued first, at clamped
  // (always valid) addresses, and masked afterwards, so no load waits behind
  // a branch or another step's MFMA.
  const int steps = (d + 31) / 32;
  // steps per load batch (the fused norm's fp64 products need registers)
  constexpr int B = NORM ? (MOE_ROUTE_UNROLL > 2 ? 2 : MOE_ROUTE_UNROLL) : MOE_ROUTE_UNROLL;
  const uint16_t* wrow[EG];
  bool e_ok[EG];
#pragma unroll
  for (int g = 0; g < EG; ++g) {
    const int e = 16 * g + (lane & 15);
    e_ok[g] = e < E;
    wrow[g] = wr + (size_t)(e_ok[g] ? e : 0) * d;
  }
  // fused RMSNorm: the factor of each of the block's 16 rows, from an fp64
  // sum of squares in a fixed order (a lane's elements, the 4 lanes of a row,
  // then the wavefronts in order)
  double rnorm = 0.0;
  if constexpr (NORM) {
    double ss = 0.0;
    for (int s0 = wv; s0 < steps; s0 += B * kMfmaWaves) {
      bf16x8_t xv[B];
      bool okn[B];
#pragma unroll
      for (int u = 0; u < B; ++u) {
        const int k = 32 * (s0 + u * kMfmaWaves) + 8 * kg;
        okn[u] = k < d;
        xv[u] = load_bf16x8(xr + (okn[u] ? k : 0));
      }
#pragma unroll
      for (int u = 0; u < B; ++u)
        if (okn[u]) ss = sumsq8(xv[u], ss);
    }
    ss += __shfl_xor(ss, 16, 64);
    ss += __shfl_xor(ss, 32, 64);
    if (lane < 16) ssq[wv][lane] = ss;
    __syncthreads();
    double tot = 0.0;
    for (int w = 0; w < kMfmaWaves; ++w) tot += ssq[w][lane & 15];
    rnorm = 1.0 / sqrt(tot / d + static_cast<double>(a.eps));
  }
  for (int s0 = wv; s0 < steps; s0 += B * kMfmaWaves) {
    bf16x8_t av[B], bv[B][EG];
    bool ok[B];
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const int k = 32 * (s0 + u * kMfmaWaves) + 8 * kg;
      ok[u] = k < d;  // d % 8 == 0: a lane's 8 elements are all in or all out
      const int kc = ok[u] ? k : 0;
      av[u] = load_bf16x8(xr + kc);
#pragma unroll
      for (int g = 0; g < EG; ++g) bv[u][g] = load_bf16x8(wrow[g] + kc);
    }
    if constexpr (NORM) {
      // each (row, 8 elements) belongs to one lane of one wavefront: it
      // normalises them, feeds them to the logits and stores them once
#pragma unroll
      for (int u = 0; u < B; ++u) {
        const int k = 32 * (s0 + u * kMfmaWaves) + 8 * kg;
        av[u] = rms_scale8(av[u], rnorm, a.norm_w + (ok[u] ? k : 0));
        if (tok_ok && ok[u]) *reinterpret_cast<bf16x8_t*>(a.xn + (size_t)tok * d + k) = av[u];
      }
    }
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const bf16x8_t a_u = (tok_ok && ok[u]) ? av[u] : zero_bf16x8();
#pragma unroll
      for (int g = 0; g < EG; ++g) acc[g] = mfma_16x16x32(a_u, e_ok[g] ? bv[u][g] : zero_bf16x8(), acc[g]);
    }
  }
  if constexpr (TREE) {
    // fixed pairwise tree: in round n, waves n/2 .. n-1 hand their tiles to
    // waves 0 .. n/2-1, which add them to their own
#pragma unroll
    for (int n = WAVES; n > 1; n /= 2) {
      if (wv >= n / 2 && wv < n) {
#pragma unroll
        for (int g = 0; g < EG; ++g)
#pragma unroll
          for (int r = 0; r < 4; ++r) part[wv - n / 2][(g * 4 + r) * 64 + lane] = acc[g][r];
      }
      __syncthreads();
      if (wv < n / 2) {
#pragma unroll
        for (int g = 0; g < EG; ++g)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[g][r] += part[wv][(g * 4 + r) * 64 + lane];
      }
      __syncthreads();
    }
    if (wv == 0) {
#pragma unroll
      for (int g = 0; g < EG; ++g)
#pragma unroll
        for (int r = 0; r < 4; ++r) lg[4 * kg + r][16 * g + (lane & 15)] = acc[g][r];
    }
    __syncthreads();
  } else {
    // partial tiles added in wavefront order
    for (int w = 0; w < kMfmaWaves; ++w) {
      if (wv == w) {
#pragma unroll
        for (int g = 0; g < EG; ++g)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = 4 * kg + r, col = 16 * g + (lane & 15);
            lg[row][col] = (w == 0) ? acc[g][r] : lg[row][col] + acc[g][r];
          }
      }
      __syncthreads();
    }
  }
  for (int i = tid; i < kMfmaTokens * E; i += 64 * kMfmaWaves) {
    const int r = i / E, e = i % E;
    if (a.br) lg[r][e] += bf16_to_f32(static_cast<const uint16_t*>(a.br)[e]);
  }
  __syncthreads();
  constexpr int VPL = (EP + 63) / 64;
  for (int r = wv; r < kMfmaTokens; r += kMfmaWaves) {
    const int t = t0 + r;
    if (t < a.T) choose_experts<VPL>(a, lg[r], t, lane, cnt);
  }
  __syncthreads();
  for (int e = tid; e < E; e += 64 * kMfmaWaves) a.hist[(size_t)blk * E + e] = cnt[e];
}

}  // namespace
}  // namespace moe
