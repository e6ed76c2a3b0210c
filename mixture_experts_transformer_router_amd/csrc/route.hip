// Router: logits, expert choice and routing weights, plus per-block expert
// counts for the permutation.
//
// Logits l[t,e] = sum_i x[t,i] Wr[e,i] + br[e] are accumulated in fp32 over i
// in increasing order (router kernel and bias: MaxText GPT-OSS weight mapping,
// "MoE Router"; glm4_moe_lite.go, MoEGate.Forward).  Each block owns 64
// tokens; its 256 threads hold a [64 tokens x E] tile of logits in registers
// while the input dimension streams through LDS in chunks of 32.
//
// Choice: one wavefront per token at a time; lane l holds the scores of
// experts l, l+64, ...; k rounds of a wave arg-max by (score desc, index asc)
// pick the experts best first.
//   GPT-OSS:  score = logit, w = softmax over the k chosen logits.
//   grouped:  s = softmax(l) over E (or sigmoid(l)), s' = s + correction bias,
//             group score = max s' in each of n_group contiguous groups, the
//             topk_group best groups are kept, top-k by s' among them,
//             w = s[chosen], renormalised if k > 1 and norm, times rsf
//             (glm4_moe_lite.go: Config n_group/topk_group, MoEGate.Forward).
#include "device_common.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 32;

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
};

// EPT = experts per thread (E <= 4 * EPT); TIn = float or uint16_t (bf16).
template <typename TIn, int EPT>
__global__ __launch_bounds__(kThreads) void route_kernel(RouteArgs a) {
  __shared__ float xs[kRouteTokens][kChunk + 1];
  __shared__ float ws[4 * EPT][kChunk + 1];
  __shared__ float lg[kRouteTokens][4 * EPT + 1];
  __shared__ int cnt[4 * EPT];

  const TIn* x = static_cast<const TIn*>(a.x);
  const TIn* wr = static_cast<const TIn*>(a.wr);
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * kRouteTokens;
  const int my_tok = tid & 63;
  const int egrp = tid >> 6;  // experts egrp, egrp + 4, ...
  const int E = a.E, d = a.d;

  for (int e = tid; e < 4 * EPT; e += kThreads) cnt[e] = 0;

  float acc[EPT];
#pragma unroll
  for (int j = 0; j < EPT; ++j) acc[j] = 0.f;

  for (int c0 = 0; c0 < d; c0 += kChunk) {
    for (int i = tid; i < kRouteTokens * kChunk; i += kThreads) {
      int r = i / kChunk, c = i % kChunk;
      int t = t0 + r;
      xs[r][c] = (t < a.T && c0 + c < d) ? load_f32(x, (size_t)t * d + c0 + c) : 0.f;
    }
    for (int i = tid; i < 4 * EPT * kChunk; i += kThreads) {
      int e = i / kChunk, c = i % kChunk;
      ws[e][c] = (e < E && c0 + c < d) ? load_f32(wr, (size_t)e * d + c0 + c) : 0.f;
    }
    __syncthreads();
#pragma unroll 4
    for (int c = 0; c < kChunk; ++c) {
      float xv = xs[my_tok][c];
#pragma unroll
      for (int j = 0; j < EPT; ++j) acc[j] = fmaf(xv, ws[egrp + 4 * j][c], acc[j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    int e = egrp + 4 * j;
    float b = (a.br != nullptr && e < E) ? load_f32(static_cast<const TIn*>(a.br), e) : 0.f;
    lg[my_tok][e] = acc[j] + b;
  }
  __syncthreads();

  // ---- choice: wave `wv` handles tokens wv, wv+4, ...
  const int lane = tid & 63, wv = tid >> 6;
  constexpr int VPL = (4 * EPT + 63) / 64;  // values per lane
  for (int r = wv; r < kRouteTokens; r += 4) {
    const int t = t0 + r;
    if (t >= a.T) break;
    float sc[VPL];     // selection score
    float base[VPL];   // weight source (logit for GPT-OSS, s for grouped)
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      int e = lane + 64 * v;
      const float l = e < E ? lg[r][e] : -INFINITY;
      sc[v] = l != l ? -INFINITY : l;  // NaN never outranks a number
    }
    bool allowed[VPL];
#pragma unroll
    for (int v = 0; v < VPL; ++v) allowed[v] = (lane + 64 * v) < E;

    if (a.grouped) {
      // scores
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
        int e = lane + 64 * v;
        float sel = base[v] + ((a.e_bias != nullptr && e < E) ? a.e_bias[e] : 0.f);
        sc[v] = (allowed[v] && sel == sel) ? sel : -INFINITY;
        if (e < E) lg[r][e] = sc[v];  // selection scores, read back per group below
      }
      // group scores: lane g < n_group takes the max over its contiguous group
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      const int gsz = E / a.n_group;
      float gscore = -INFINITY;
      int gidx = kNoIndex;
      if (lane < a.n_group) {
        for (int i = 0; i < gsz; ++i) gscore = fmaxf(gscore, lg[r][lane * gsz + i]);
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
        int e = lane + 64 * v;
        if (e < E && !((kept >> (e / gsz)) & 1ull)) allowed[v] = false;
      }
    } else {
#pragma unroll
      for (int v = 0; v < VPL; ++v) base[v] = sc[v];
    }

    // k rounds of arg-max over the allowed experts
    int my_e = -1;
    float my_base = 0.f, first_base = 0.f;
    for (int j = 0; j < a.k; ++j) {
      float bv = -INFINITY;
      int bi = kNoIndex;
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        int e = lane + 64 * v;
        if (allowed[v] && precedes(sc[v], e, bv, bi)) { bv = sc[v]; bi = e; }
      }
      wave_argmax(bv, bi);
      // the host guarantees at least k allowed experts, so bi < E here
      // owner lane of expert bi retires it and broadcasts its weight source
      float bb = 0.f;
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        if (lane + 64 * v == bi) { allowed[v] = false; bb = base[v]; }
      }
      bb = __shfl(bb, bi & 63, 64);
      if (j == 0) first_base = bb;
      if (lane == j) { my_e = bi; my_base = bb; }
    }
    // weights
    float wv_ = 0.f;
    if (!a.grouped) {
      float ex = lane < a.k ? expf(my_base - first_base) : 0.f;
      float s = wave_sum(ex);
      wv_ = ex / s;
    } else {
      wv_ = lane < a.k ? my_base : 0.f;
      if (a.k > 1 && a.norm) {
        float s = wave_sum(wv_);
        wv_ = wv_ / s;
      }
      wv_ *= a.rsf;
    }
    if (lane < a.k) {
      size_t o = (size_t)t * a.k + lane;
      a.idx[o] = my_e;
      a.w[o] = wv_;
      if (a.user_idx) a.user_idx[o] = my_e;
      if (a.user_w) a.user_w[o] = wv_;
      atomicAdd(&cnt[my_e], 1);
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += kThreads) a.hist[(size_t)blockIdx.x * E + e] = cnt[e];
}

template <typename TIn>
hipError_t launch_t(const RouteArgs& a, int nblk, hipStream_t s) {
  if (a.E <= 8) route_kernel<TIn, 2><<<nblk, kThreads, 0, s>>>(a);
  else if (a.E <= 16) route_kernel<TIn, 4><<<nblk, kThreads, 0, s>>>(a);
  else if (a.E <= 32) route_kernel<TIn, 8><<<nblk, kThreads, 0, s>>>(a);
  else if (a.E <= 64) route_kernel<TIn, 16><<<nblk, kThreads, 0, s>>>(a);
  else route_kernel<TIn, 64><<<nblk, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const Layer& L, const Work& W, hipStream_t s) {
  RouteArgs a;
  a.x = L.x; a.wr = L.router_w; a.br = L.router_b; a.e_bias = L.e_bias;
  a.T = L.T; a.d = L.d; a.E = L.E; a.k = L.k;
  a.grouped = L.grouped; a.n_group = L.n_group; a.topk_group = L.topk_group;
  a.norm = L.norm; a.score = L.score; a.rsf = L.rsf;
  a.idx = W.idx; a.w = W.w; a.hist = W.hist;
  a.user_idx = L.routing.topk_idx; a.user_w = L.routing.topk_w;
  int nblk = (L.T + kRouteTokens - 1) / kRouteTokens;
  return L.dt == MOE_F32 ? launch_t<float>(a, nblk, s) : launch_t<uint16_t>(a, nblk, s);
}

}  // namespace moe
