// Router arguments and the per-token expert choice, shared by the router
// kernels and the few-token choose-and-permute kernel.  (Device code of one
// translation unit each: this header is included by route.hip and permute.hip.)
//
// Choice: one wavefront per token; lane l holds the scores of experts l,
// l+64, ...; k rounds of a wave arg-max by (score desc, index asc) pick the
// experts best first.
//   GPT-OSS:  score = logit, w = softmax over the k chosen logits.
//   grouped:  s = softmax(l) over E (or sigmoid(l)), s' = s + correction bias,
//             group score = max s' in each of n_group contiguous groups, the
//             topk_group best groups are kept, top-k by s' among them,
//             w = s[chosen], renormalised if k > 1 and norm, times rsf
//             (glm4_moe_lite.go: Config n_group/topk_group, MoEGate.Forward).
#pragma once

#include "device_common.h"
#include "moe_internal.h"

namespace moe {
namespace {

struct RouteArgs {
  const void* x;
  const void* wr;
  const void* br;
  const float* e_bias;
  int T, d, E, k;
  int grouped, n_group, topk_group, norm, score;
  float rsf;
  int32_t* idx;
  float* w;
  int32_t* hist;
  int32_t* user_idx;
  float* user_w;
  // MoE block, bf16: RMSNorm of the rows fused into the router (nullptr: no
  // norm).  The router computes each row's factor, feeds the normalised rows
  // to its logits and writes them to xn for the expert stages.
  const uint16_t* norm_w;
  float eps;
  uint16_t* xn;
};

// Fused RMSNorm (glm4_moe_lite.go, MoEBlock.Forward: PostAttentionLayerNorm):
// 8 consecutive elements x[k .. k+7] of a row with factor r (the row's
// 1 / sqrt(mean(x^2) + eps), fp64) become x * r * w rounded once from fp64 to
// bf16 -- the same expression and rounding as the stand-alone norm kernel.
__device__ __forceinline__ bf16x8_t rms_scale8(bf16x8_t xv, double r, const uint16_t* w8) {
  const u32x4_t xw = __builtin_bit_cast(u32x4_t, xv);
  const u32x4_t ww = *reinterpret_cast<const u32x4_t*>(w8);
  u32x4_t o;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t xp = xw[i], wp = ww[i];
    const uint16_t lo = f64_to_bf16(static_cast<double>(bf16_to_f32(xp & 0xffffu)) * r *
                                    static_cast<double>(bf16_to_f32(wp & 0xffffu)));
    const uint16_t hi = f64_to_bf16(static_cast<double>(bf16_to_f32(xp >> 16)) * r *
                                    static_cast<double>(bf16_to_f32(wp >> 16)));
    o[i] = static_cast<uint32_t>(lo) | (static_cast<uint32_t>(hi) << 16);
  }
  return __builtin_bit_cast(bf16x8_t, o);
}

// fp64 sum of squares of 8 bf16 elements added to ss in element order
__device__ __forceinline__ double sumsq8(bf16x8_t xv, double ss) {
  const u32x4_t xw = __builtin_bit_cast(u32x4_t, xv);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const double lo = bf16_to_f32(xw[i] & 0xffffu), hi = bf16_to_f32(xw[i] >> 16);
    ss = fma(lo, lo, ss);
    ss = fma(hi, hi, ss);
  }
  return ss;
}

// Choose the experts of token t from its logits row `lg` (LDS, E entries;
// overwritten with selection scores on the grouped path) with one wavefront.
// VPL = experts per lane (E <= 64 * VPL).  Adds the chosen experts to `cnt`
// and, if `chosen` is given, stores them there (best first, k entries).
template <int VPL>
__device__ void choose_experts(const RouteArgs& a, float* lg, int t, int lane, int* cnt, int* chosen = nullptr) {
  const int E = a.E;
  float sc[VPL];    // selection score
  float base[VPL];  // weight source (logit for GPT-OSS, s for grouped)
  bool allowed[VPL];
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    const int e = lane + 64 * v;
    const float l = e < E ? lg[e] : -INFINITY;
    sc[v] = l != l ? -INFINITY : l;  // NaN never outranks a number
    allowed[v] = e < E;
  }

  if (a.grouped) {
    if (a.score == MOE_SCORE_SOFTMAX) {
      float m = -INFINITY;
#pragma unroll
      for (int v = 0; v < VPL; ++v) m = fmaxf(m, sc[v]);
      m = wave_max(m);
      float s = 0.f;
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        base[v] = allowed[v] ? expf(sc[v] - m) : 0.f;
        s += base[v];
      }
      s = wave_sum(s);
#pragma unroll
      for (int v = 0; v < VPL; ++v) base[v] = base[v] / s;
    } else {
#pragma unroll
      for (int v = 0; v < VPL; ++v) base[v] = allowed[v] ? 1.0f / (1.0f + expf(-sc[v])) : 0.f;
    }
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      const int e = lane + 64 * v;
      const float sel = base[v] + ((a.e_bias != nullptr && e < E) ? a.e_bias[e] : 0.f);
      sc[v] = (allowed[v] && sel == sel) ? sel : -INFINITY;
      if (e < E) lg[e] = sc[v];  // read back per group below (same wavefront)
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // group scores: lane g < n_group takes the max over its contiguous group
    const int gsz = E / a.n_group;
    float gscore = -INFINITY;
    int gidx = kNoIndex;
    if (lane < a.n_group) {
      for (int i = 0; i < gsz; ++i) gscore = fmaxf(gscore, lg[lane * gsz + i]);
      gidx = lane;
    }
    uint64_t kept = 0;
    for (int j = 0; j < a.topk_group; ++j) {
      float bv = gscore;
      int bi = gidx;
      wave_argmax(bv, bi);
      kept |= 1ull << bi;
      if (lane == bi) { gscore = -INFINITY; gidx = kNoIndex; }
    }
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      const int e = lane + 64 * v;
      if (e < E && !((kept >> (e / gsz)) & 1ull)) allowed[v] = false;
    }
  } else {
#pragma unroll
    for (int v = 0; v < VPL; ++v) base[v] = sc[v];
  }

  // k rounds of arg-max over the allowed experts; the host guarantees at
  // least k allowed experts, so every round finds one (bi < E).
  int my_e = -1;
  float my_base = 0.f, first_base = 0.f;
  for (int j = 0; j < a.k; ++j) {
    float bv = -INFINITY;
    int bi = kNoIndex;
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      const int e = lane + 64 * v;
      if (allowed[v] && precedes(sc[v], e, bv, bi)) { bv = sc[v]; bi = e; }
    }
    wave_argmax(bv, bi);
    float bb = 0.f;
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      if (lane + 64 * v == bi) { allowed[v] = false; bb = base[v]; }
    }
    bb = __shfl(bb, bi & 63, 64);
    if (j == 0) first_base = bb;
    if (lane == j) { my_e = bi; my_base = bb; }
  }
  float wt;
  if (!a.grouped) {
    const float ex = lane < a.k ? expf(my_base - first_base) : 0.f;
    wt = ex / wave_sum(ex);
  } else {
    wt = lane < a.k ? my_base : 0.f;
    if (a.k > 1 && a.norm) wt = wt / wave_sum(wt);
    wt *= a.rsf;
  }
  if (lane < a.k) {
    const size_t o = (size_t)t * a.k + lane;
    a.idx[o] = my_e;
    a.w[o] = wt;
    if (a.user_idx) a.user_idx[o] = my_e;
    if (a.user_w) a.user_w[o] = wt;
    atomicAdd(&cnt[my_e], 1);
    if (chosen) chosen[lane] = my_e;
  }
}

// The few-token path (bf16, T <= kDecodeMaxTokens): split-K router logits,
// then one kernel that chooses the experts and permutes.
inline bool few_token_route(const Layer& L) { return L.dt != MOE_F32 && L.T <= kDecodeMaxTokens; }

inline RouteArgs route_args(const Layer& L, const Work& W) {
  RouteArgs a;
  a.x = L.x; a.wr = L.router_w; a.br = L.router_b; a.e_bias = L.e_bias;
  a.T = L.T; a.d = L.d; a.E = L.E; a.k = L.k;
  a.grouped = L.grouped; a.n_group = L.n_group; a.topk_group = L.topk_group;
  a.norm = L.norm; a.score = L.score; a.rsf = L.rsf;
  a.idx = W.idx; a.w = W.w; a.hist = W.hist;
  a.user_idx = L.routing.topk_idx; a.user_w = L.routing.topk_w;
  const bool fuse_norm = L.norm_w != nullptr && L.dt == MOE_BF16 && !few_token_route(L);
  a.norm_w = fuse_norm ? static_cast<const uint16_t*>(L.norm_w) : nullptr;
  a.eps = L.eps;
  a.xn = fuse_norm ? static_cast<uint16_t*>(W.xn) : nullptr;
  return a;
}


}  // namespace
}  // namespace moe
