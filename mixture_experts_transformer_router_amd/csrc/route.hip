// Router: logits, expert choice and routing weights, plus per-block expert
// counts for the permutation.
//
// Logits l[t,e] = sum_i x[t,i] Wr[e,i] + br[e], accumulated in fp32 (router
// kernel and bias: MaxText GPT-OSS weight mapping, "MoE Router";
// glm4_moe_lite.go, MoEGate.Forward).
//   bf16: a [16 tokens x 16 experts] tile per MFMA; the block's wavefronts
//         split the input dimension and their partial tiles are added in a
//         fixed order (deterministic).  For T <= 16 the input dimension is
//         also split over blocks (route_split_logits_kernel); the permute
//         stage adds the slices in order and chooses.
//   fp32: 64 tokens per block on the vector ALUs, the input dimension
//         streaming through LDS in chunks of 32.
// MoE block (bf16, many tokens): the RMSNorm in front of the layer is fused
// into route_mfma_kernel.  A block first sums the squares of its 16 rows in
// fp64, then normalises each 8-element piece as it loads it for the logits
// (x * r * w, rounded once to bf16) and stores the normalised rows for the
// expert stages: x is not read by a norm kernel of its own, and xn is not
// read back by the router.  (For T <= 16 the split router would need every
// whole row in each of its blocks; the stand-alone norm kernel runs first.)
//
// Choice: see route_common.h.
#include "route_mfma.h"

namespace moe {
namespace {

// One block per 16 tokens.
template <int EG, int WAVES, bool TREE, bool NORM>
__global__ __launch_bounds__(64 * WAVES) void route_mfma_kernel(RouteArgs a) {
  route_mfma_block<EG, WAVES, TREE, NORM>(a, blockIdx.x);
}

// ---- bf16, few tokens (T <= 16): split-K logits, then the choice --------------
// A single block would read the whole router through one CU's memory
// pipeline; here block (g, ks) computes the [16 tokens x 16 experts] tile of
// expert group g over the ks-th of kRouteSplitK contiguous slices of the input
// dimension (one wavefront, all loads of a slice issued before its MFMAs) and
// stores it to part[ks].  select_permute_small_kernel (permute.hip) adds the
// slices in ks order and chooses.
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

template <bool NORM>
void launch_mfma_router(const RouteArgs& a, int E, int nblk, bool wide, hipStream_t s) {
  // Fewer blocks than CUs (latency-bound): up to 64 experts take 16
  // wavefronts and a tree sum.  Otherwise 8 wavefronts in wavefront order
  // (more blocks resident per CU).
  if (wide) {
    if (E <= 16) route_mfma_kernel<1, 16, true, NORM><<<nblk, 64 * 16, 0, s>>>(a);
    else if (E <= 32) route_mfma_kernel<2, 16, true, NORM><<<nblk, 64 * 16, 0, s>>>(a);
    else route_mfma_kernel<4, 16, true, NORM><<<nblk, 64 * 16, 0, s>>>(a);
  } else {
    if (E <= 16) route_mfma_kernel<1, 8, false, NORM><<<nblk, 64 * 8, 0, s>>>(a);
    else if (E <= 32) route_mfma_kernel<2, 8, false, NORM><<<nblk, 64 * 8, 0, s>>>(a);
    else if (E <= 64) route_mfma_kernel<4, 8, false, NORM><<<nblk, 64 * 8, 0, s>>>(a);
    else if (E <= 128) route_mfma_kernel<8, 8, false, NORM><<<nblk, 64 * 8, 0, s>>>(a);
    else route_mfma_kernel<16, 8, false, NORM><<<nblk, 64 * 8, 0, s>>>(a);
  }
}

}  // namespace

int route_block_tokens(const Layer& L) { return L.dt == MOE_F32 ? kValuTokens : kMfmaTokens; }

hipError_t launch_route(const Layer& L, const Work& W, hipStream_t s) {
  const RouteArgs a = route_args(L, W);
  if (few_token_route(L)) {
    // the choice runs in the permute stage (select_permute_small_kernel)
    route_split_logits_kernel<<<dim3((L.E + 15) / 16, kRouteSplitK), 64, 0, s>>>(a, W.route_part);
    return hipGetLastError();
  }
  const int tb = route_block_tokens(L);
  const int nblk = (L.T + tb - 1) / tb;
  if (L.dt == MOE_F32) {
    if (L.E <= 8) route_valu_kernel<2><<<nblk, kValuThreads, 0, s>>>(a);
    else if (L.E <= 16) route_valu_kernel<4><<<nblk, kValuThreads, 0, s>>>(a);
    else if (L.E <= 32) route_valu_kernel<8><<<nblk, kValuThreads, 0, s>>>(a);
    else if (L.E <= 64) route_valu_kernel<16><<<nblk, kValuThreads, 0, s>>>(a);
    else route_valu_kernel<64><<<nblk, kValuThreads, 0, s>>>(a);
  } else {
    constexpr bool kTree = MOE_ROUTE_TREE != 0;
    const bool wide = kTree && nblk < 256 && L.E <= 64;
    if (a.norm_w) launch_mfma_router<true>(a, L.E, nblk, wide, s);
    else launch_mfma_router<false>(a, L.E, nblk, wide, s);
  }
  return hipGetLastError();
}

}  // namespace moe
