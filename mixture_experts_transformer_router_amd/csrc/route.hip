// Router: logits, expert choice and routing weights, plus per-block expert
// counts for the permutation.
//
// Logits l[t,e] = sum_i x[t,i] Wr[e,i] + br[e], accumulated in fp32 (router
// kernel and bias: MaxText GPT-OSS weight mapping, "MoE Router";
// glm4_moe_lite.go, MoEGate.Forward).
//   bf16: a [16 tokens x 16 experts] tile per MFMA; the block's wavefronts
//         split the input dimension and their partial tiles are added in a
//         fixed order (deterministic).  For T <= 16 the input dimension is
//         also split over blocks (route_split_logits_kernel) and a one-block
//         kernel adds the slices in order and chooses.
//   fp32: 64 tokens per block on the vector ALUs, the input dimension
//         streaming through LDS in chunks of 32.
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
};

// Choose the experts of token t from its logits row `lg` (LDS, E entries;
// overwritten with selection scores on the grouped path) with one wavefront.
// VPL = experts per lane (E <= 64 * VPL).  Adds the chosen experts to `cnt`.
template <int VPL>
__device__ void choose_experts(const RouteArgs& a, float* lg, int t, int lane, int* cnt) {
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
  }
}

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
template <int EG, int WAVES, bool TREE>
__global__ __launch_bounds__(64 * WAVES) void route_mfma_kernel(RouteArgs a) {
  constexpr int EP = 16 * EG;
  constexpr int kMfmaWaves = WAVES;
  __shared__ float lg[kMfmaTokens][EP + 1];
  __shared__ float part[TREE ? WAVES / 2 : 1][TREE ? EG * 4 * 64 : 1];
  __shared__ int cnt[EP];
  const uint16_t* x = static_cast<const uint16_t*>(a.x);
  const uint16_t* wr = static_cast<const uint16_t*>(a.wr);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int t0 = blockIdx.x * kMfmaTokens;
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
  constexpr int B = MOE_ROUTE_UNROLL;
  const uint16_t* wrow[EG];
  bool e_ok[EG];
#pragma unroll
  for (int g = 0; g < EG; ++g) {
    const int e = 16 * g + (lane & 15);
    e_ok[g] = e < E;
    wrow[g] = wr + (size_t)(e_ok[g] ? e : 0) * d;
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
  for (int e = tid; e < E; e += 64 * kMfmaWaves) a.hist[(size_t)blockIdx.x * E + e] = cnt[e];
}

// ---- bf16, few tokens (T <= 16): split-K logits, then the choice --------------
// A single block would read the whole router through one CU's memory
// pipeline; here block (g, ks) computes the [16 tokens x 16 experts] tile of
// expert group g over the ks-th of kRouteSplitK contiguous slices of the input
// dimension (one wavefront, all loads of a slice issued before its MFMAs) and
// stores it to part[ks].  route_choose_kernel adds the slices in ks order.
constexpr int kSplitSteps = 8;  // 32-element steps loaded ahead by one wavefront

__global__ __launch_bounds__(64) void route_split_logits_kernel(RouteArgs a, float* part) {
  const uint16_t* x = static_cast<const uint16_t*>(a.x);
  const uint16_t* wr = static_cast<const uint16_t*>(a.wr);
  const int g = blockIdx.x, ks = blockIdx.y, lane = threadIdx.x;
  const int kg = lane >> 4, d = a.d, E = a.E;
  const int tok = lane & 15, e = 16 * g + (lane & 15);
  const bool tok_ok = tok < a.T, e_ok = e < E;
  const uint16_t* xr = x + (size_t)(tok_ok ? tok : 0) * d;
  const uint16_t* wrow = wr + (size_t)(e_ok ? e : 0) * d;
  const int steps = (d + 31) / 32;
  const int s_begin = steps * ks / kRouteSplitK, s_end = steps * (ks + 1) / kRouteSplitK;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = s_begin; s0 < s_end; s0 += kSplitSteps) {
    bf16x8_t av[kSplitSteps], bv[kSplitSteps];
    bool ok[kSplitSteps];
#pragma unroll
    for (int u = 0; u < kSplitSteps; ++u) {
      const int k = 32 * (s0 + u) + 8 * kg;
      ok[u] = s0 + u < s_end && k < d;  // d % 8 == 0: a lane's 8 elements are all in or all out
      const int kc = ok[u] ? k : 0;
      av[u] = load_bf16x8(xr + kc);
      bv[u] = load_bf16x8(wrow + kc);
    }
#pragma unroll
    for (int u = 0; u < kSplitSteps; ++u)
      acc = mfma_16x16x32((tok_ok && ok[u]) ? av[u] : zero_bf16x8(), (e_ok && ok[u]) ? bv[u] : zero_bf16x8(), acc);
  }
  // lane holds tokens 4 kg .. 4 kg + 3 of expert e
  if (e_ok) {
#pragma unroll
    for (int r = 0; r < 4; ++r) part[((size_t)ks * 16 + 4 * kg + r) * E + e] = acc[r];
  }
}

// One block: logits = sum of the kRouteSplitK slices in order + bias, then one
// wavefront per token chooses its experts; writes the block's expert counts.
template <int VPL>
__global__ __launch_bounds__(1024) void route_choose_kernel(RouteArgs a, const float* part) {
  __shared__ float lg[16][64 * VPL + 1];
  __shared__ int cnt[64 * VPL];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int E = a.E;
  for (int e = tid; e < E; e += 1024) cnt[e] = 0;
  for (int i = tid; i < a.T * E; i += 1024) {
    const int t = i / E, e = i % E;
    float pv[kRouteSplitK];  // all slices loaded first, then added in order
#pragma unroll
    for (int ks = 0; ks < kRouteSplitK; ++ks) pv[ks] = part[((size_t)ks * 16 + t) * E + e];
    float v = 0.f;
#pragma unroll
    for (int ks = 0; ks < kRouteSplitK; ++ks) v += pv[ks];
    if (a.br) v += bf16_to_f32(static_cast<const uint16_t*>(a.br)[e]);
    lg[t][e] = v;
  }
  __syncthreads();
  if (wv < a.T) choose_experts<VPL>(a, lg[wv], wv, lane, cnt);
  __syncthreads();
  for (int e = tid; e < E; e += 1024) a.hist[e] = cnt[e];
}

// ---- fp32: vector-ALU logits -------------------------------------------------
constexpr int kValuTokens = 64;
constexpr int kValuThreads = 256;
constexpr int kChunk = 32;

// EPT = experts per thread (E <= 4 * EPT).
template <int EPT>
__global__ __launch_bounds__(kValuThreads) void route_valu_kernel(RouteArgs a) {
  __shared__ float xs[kValuTokens][kChunk + 1];
  __shared__ float ws[4 * EPT][kChunk + 1];
  __shared__ float lg[kValuTokens][4 * EPT + 1];
  __shared__ int cnt[4 * EPT];

  const float* x = static_cast<const float*>(a.x);
  const float* wr = static_cast<const float*>(a.wr);
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * kValuTokens;
  const int my_tok = tid & 63;
  const int egrp = tid >> 6;  // experts egrp, egrp + 4, ...
  const int E = a.E, d = a.d;

  for (int e = tid; e < 4 * EPT; e += kValuThreads) cnt[e] = 0;
  float acc[EPT];
#pragma unroll
  for (int j = 0; j < EPT; ++j) acc[j] = 0.f;

  for (int c0 = 0; c0 < d; c0 += kChunk) {
    for (int i = tid; i < kValuTokens * kChunk; i += kValuThreads) {
      const int r = i / kChunk, c = i % kChunk, t = t0 + r;
      xs[r][c] = (t < a.T && c0 + c < d) ? x[(size_t)t * d + c0 + c] : 0.f;
    }
    for (int i = tid; i < 4 * EPT * kChunk; i += kValuThreads) {
      const int e = i / kChunk, c = i % kChunk;
      ws[e][c] = (e < E && c0 + c < d) ? wr[(size_t)e * d + c0 + c] : 0.f;
    }
    __syncthreads();
#pragma unroll 4
    for (int c = 0; c < kChunk; ++c) {
      const float xv = xs[my_tok][c];
#pragma unroll
      for (int j = 0; j < EPT; ++j) acc[j] = fmaf(xv, ws[egrp + 4 * j][c], acc[j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const int e = egrp + 4 * j;
    const float b = (a.br != nullptr && e < E) ? static_cast<const float*>(a.br)[e] : 0.f;
    lg[my_tok][e] = acc[j] + b;
  }
  __syncthreads();
  const int lane = tid & 63, wv = tid >> 6;
  constexpr int VPL = (4 * EPT + 63) / 64;
  for (int r = wv; r < kValuTokens; r += 4) {
    const int t = t0 + r;
    if (t < a.T) choose_experts<VPL>(a, lg[r], t, lane, cnt);
  }
  __syncthreads();
  for (int e = tid; e < E; e += kValuThreads) a.hist[(size_t)blockIdx.x * E + e] = cnt[e];
}

}  // namespace

int route_block_tokens(const Layer& L) { return L.dt == MOE_F32 ? kValuTokens : kMfmaTokens; }

hipError_t launch_route(const Layer& L, const Work& W, hipStream_t s) {
  RouteArgs a;
  a.x = L.x; a.wr = L.router_w; a.br = L.router_b; a.e_bias = L.e_bias;
  a.T = L.T; a.d = L.d; a.E = L.E; a.k = L.k;
  a.grouped = L.grouped; a.n_group = L.n_group; a.topk_group = L.topk_group;
  a.norm = L.norm; a.score = L.score; a.rsf = L.rsf;
  a.idx = W.idx; a.w = W.w; a.hist = W.hist;
  a.user_idx = L.routing.topk_idx; a.user_w = L.routing.topk_w;
  const int tb = route_block_tokens(L);
  const int nblk = (L.T + tb - 1) / tb;
  if (L.dt == MOE_F32) {
    if (L.E <= 8) route_valu_kernel<2><<<nblk, kValuThreads, 0, s>>>(a);
    else if (L.E <= 16) route_valu_kernel<4><<<nblk, kValuThreads, 0, s>>>(a);
    else if (L.E <= 32) route_valu_kernel<8><<<nblk, kValuThreads, 0, s>>>(a);
    else if (L.E <= 64) route_valu_kernel<16><<<nblk, kValuThreads, 0, s>>>(a);
    else route_valu_kernel<64><<<nblk, kValuThreads, 0, s>>>(a);
  } else if (L.T <= kDecodeMaxTokens) {
    route_split_logits_kernel<<<dim3((L.E + 15) / 16, kRouteSplitK), 64, 0, s>>>(a, W.route_part);
    if (L.E <= 64) route_choose_kernel<1><<<1, 1024, 0, s>>>(a, W.route_part);
    else if (L.E <= 128) route_choose_kernel<2><<<1, 1024, 0, s>>>(a, W.route_part);
    else route_choose_kernel<4><<<1, 1024, 0, s>>>(a, W.route_part);
  } else {
    // Fewer blocks than CUs (latency-bound): up to 64 experts take 16
    // wavefronts and a tree sum.  Otherwise 8 wavefronts in wavefront order
    // (more blocks resident per CU).
    constexpr bool kTree = MOE_ROUTE_TREE != 0;
    const bool wide = kTree && nblk < 256 && L.E <= 64;
    if (wide) {
      if (L.E <= 16) route_mfma_kernel<1, 16, true><<<nblk, 64 * 16, 0, s>>>(a);
      else if (L.E <= 32) route_mfma_kernel<2, 16, true><<<nblk, 64 * 16, 0, s>>>(a);
      else route_mfma_kernel<4, 16, true><<<nblk, 64 * 16, 0, s>>>(a);
    } else {
      if (L.E <= 16) route_mfma_kernel<1, 8, false><<<nblk, 64 * 8, 0, s>>>(a);
      else if (L.E <= 32) route_mfma_kernel<2, 8, false><<<nblk, 64 * 8, 0, s>>>(a);
      else if (L.E <= 64) route_mfma_kernel<4, 8, false><<<nblk, 64 * 8, 0, s>>>(a);
      else if (L.E <= 128) route_mfma_kernel<8, 8, false><<<nblk, 64 * 8, 0, s>>>(a);
      else route_mfma_kernel<16, 8, false><<<nblk, 64 * 8, 0, s>>>(a);
    }
  }
  return hipGetLastError();
}

}  // namespace moe
