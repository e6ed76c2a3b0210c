// Permutation of the (token, slot) pairs into expert order.
//
// Pair p = t*k + j is routed to expert idx[p].  Rows of the grouped GEMMs are
// the pairs sorted by (expert, p) -- the stable sort of the flattened expert
// indices that glm4_moe_lite.go's SwitchMLP.Forward performs, with its
// inverse (pos) used to return to token order.  With a shared expert, its T
// rows (one per token, in token order) follow all routed rows.
//
// One block per 64 tokens (64*k pairs).  Each block
//   1. sums the per-router-block expert counts: totals give the expert
//      offsets (exclusive prefix sum), the counts of earlier tokens give this
//      block's first row inside each expert;
//   2. ranks its own pairs stably: per wavefront, the lanes routed to the same
//      expert are found with 9 ballots over the expert id bits; earlier
//      wavefronts and rounds are added through small LDS counters;
//   3. writes sorted_pair, row_token and pos.
// Block 0 also writes the expert offsets and the M-tile prefix used by the
// grouped GEMMs.  No atomics touch global memory: the result is unique.
#include "route_common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxE = 257;  // 256 routed experts + shared

struct PermuteArgs {
  const int32_t* idx;
  const int32_t* hist;  // [n_hist, E] expert counts per router block
  int n_hist;           // router blocks
  int hist_per_block;   // router blocks per permute block (64 / router block tokens)
  int T, k, E, shared;
  int tile_m, tile_m_big;
  int32_t* offsets;
  int32_t* tile_prefix;
  int32_t* tile_prefix_big;
  int32_t* tile_desc;
  int32_t* sorted_pair;
  int32_t* row_token;
  int32_t* pos;
  int32_t* user_offsets;
  int32_t* user_sorted;
};

__global__ __launch_bounds__(kThreads) void permute_kernel(PermuteArgs a) {
  __shared__ int total[kMaxE];
  __shared__ int before[kMaxE];
  __shared__ int off[kMaxE + 1];
  __shared__ int running[kMaxE];
  __shared__ int wcnt[4][kMaxE];
  __shared__ int tpb[kMaxE + 1];  // 256-row tile prefix (block 0)

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int b = blockIdx.x;
  const int E = a.E;

  // Column sums of the count table, split over all threads: thread
  // (part, e) adds rows part, part + parts, ... of expert e.
  {
    int* part_tot = &wcnt[0][0];           // scratch, cleared again below
    int* part_bef = &wcnt[2][0];
    const int parts = E >= kThreads ? 1 : kThreads / E;
    const int first_own = b * a.hist_per_block;
    for (int t = tid; t < parts * E; t += kThreads) {
      const int e = t % E, part = t / E;
      int tot = 0, bef = 0;
#pragma unroll 4
      for (int i = part; i < a.n_hist; i += parts) {
        const int c = a.hist[(size_t)i * E + e];
        tot += c;
        bef += i < first_own ? c : 0;
      }
      part_tot[t] = tot;
      part_bef[t] = bef;
    }
    __syncthreads();
    for (int e = tid; e < E; e += kThreads) {
      int tot = 0, bef = 0;
      for (int p = 0; p < parts; ++p) {
        tot += part_tot[p * E + e];
        bef += part_bef[p * E + e];
      }
      total[e] = tot;
      before[e] = bef;
      running[e] = 0;
    }
    __syncthreads();
  }
  for (int i = tid; i < 4 * kMaxE; i += kThreads) (&wcnt[0][0])[i] = 0;
  __syncthreads();
  if (tid == 0) {
    int acc = 0;
    for (int e = 0; e < E; ++e) { off[e] = acc; acc += total[e]; }
    off[E] = acc;
  }
  __syncthreads();

  if (b == 0) {
    const int Eall = E + (a.shared ? 1 : 0);
    for (int e = tid; e <= E; e += kThreads) {
      a.offsets[e] = off[e];
      if (a.user_offsets) a.user_offsets[e] = off[e];
    }
    if (a.shared && tid == 0) a.offsets[E + 1] = off[E] + a.T;
    if (tid == 0) {
      int acc = 0, acc_big = 0;
      for (int e = 0; e < Eall; ++e) {
        a.tile_prefix[e] = acc;
        a.tile_prefix_big[e] = acc_big;
        tpb[e] = acc_big;
        const int c = e < E ? total[e] : a.T;
        acc += (c + a.tile_m - 1) / a.tile_m;
        acc_big += (c + a.tile_m_big - 1) / a.tile_m_big;
      }
      a.tile_prefix[Eall] = acc;
      a.tile_prefix_big[Eall] = acc_big;
      tpb[Eall] = acc_big;
    }
    __syncthreads();
    // one descriptor per 256-row tile: {expert, first row, end row, 0}
    for (int e = tid; e < Eall; e += kThreads) {
      const int first = tpb[e];
      const int n = tpb[e + 1] - first;
      const int r_begin = e < E ? off[e] : off[E];
      const int r_end = e < E ? off[e + 1] : off[E] + a.T;
      for (int j = 0; j < n; ++j) {
        int32_t* d = a.tile_desc + 4 * (size_t)(first + j);
        d[0] = e;
        d[1] = r_begin + j * a.tile_m_big;
        d[2] = r_end;
        d[3] = 0;
      }
    }
  }

  const int t_begin = b * kPermuteTokens;
  const int t_end = min(a.T, t_begin + kPermuteTokens);
  const int p_begin = t_begin * a.k;
  const int n = (t_end - t_begin) * a.k;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

  for (int r0 = 0; r0 < n; r0 += kThreads) {
    const int pl = r0 + tid;
    const bool valid = pl < n;
    const int e = valid ? a.idx[p_begin + pl] : 0;
    uint64_t m = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < 9; ++bit) {
      const bool on = (e >> bit) & 1;
      const uint64_t bm = __ballot(on);
      m &= on ? bm : ~bm;
    }
    const int rank = __popcll(m & lt_mask);
    if (valid && rank == 0) wcnt[wv][e] = __popcll(m);
    __syncthreads();
    if (valid) {
      int pre = running[e];
      for (int w2 = 0; w2 < wv; ++w2) pre += wcnt[w2][e];
      const int dest = off[e] + before[e] + pre + rank;
      const int p = p_begin + pl;
      a.sorted_pair[dest] = p;
      a.row_token[dest] = p / a.k;
      a.pos[p] = dest;
      if (a.user_sorted) a.user_sorted[dest] = p;
    }
    __syncthreads();
    for (int ee = tid; ee < E; ee += kThreads) {
      running[ee] += wcnt[0][ee] + wcnt[1][ee] + wcnt[2][ee] + wcnt[3][ee];
      wcnt[0][ee] = wcnt[1][ee] = wcnt[2][ee] = wcnt[3][ee] = 0;
    }
    __syncthreads();
  }

  if (a.shared) {
    const int P = a.T * a.k;
    for (int t = t_begin + tid; t < t_end; t += kThreads) {
      a.sorted_pair[P + t] = -1;
      a.row_token[P + t] = t;
    }
  }
}

// ---- few tokens (bf16, T <= 16): choose the experts and permute in one block --
// Logits = the router's kRouteSplitK partial slices added in order + bias;
// wavefront t chooses token t's experts (choose_experts: writes idx, w and
// the routing outputs).  The block then holds every pair's expert and the
// per-expert counts, so no count table goes through global memory: wavefront
// 0 scans the counts into offsets and tile prefixes, one thread per expert
// writes its tile descriptors, and thread p ranks pair p among the earlier
// pairs of its expert (stable, so the order is the same as permute_kernel's).
template <int VPL>
__global__ __launch_bounds__(1024) void select_permute_small_kernel(RouteArgs ra, PermuteArgs a, const float* part) {
  constexpr int EP = 64 * VPL;
  __shared__ float lg[kDecodeMaxTokens][EP + 1];
  __shared__ int cnt[EP];
  __shared__ int chosen[kDecodeMaxTokens * 16];  // pair p = t * k + j
  __shared__ int off[EP + 2];                    // routed experts, then the shared one
  __shared__ int tpb[EP + 2];                    // 256-row tile prefix
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int E = ra.E, T = ra.T, k = ra.k, P = T * k;
  for (int e = tid; e < EP; e += 1024) cnt[e] = 0;
  for (int i = tid; i < T * E; i += 1024) {
    const int t = i / E, e = i % E;
    float pv[kRouteSplitK];  // all slices loaded first, then added in order
#pragma unroll
    for (int ks = 0; ks < kRouteSplitK; ++ks) pv[ks] = part[((size_t)ks * 16 + t) * E + e];
    float v = 0.f;
#pragma unroll
    for (int ks = 0; ks < kRouteSplitK; ++ks) v += pv[ks];
    if (ra.br) v += bf16_to_f32(static_cast<const uint16_t*>(ra.br)[e]);
    lg[t][e] = v;
  }
  __syncthreads();
  if (wv < T) choose_experts<VPL>(ra, lg[wv], wv, lane, cnt, &chosen[wv * k]);
  __syncthreads();

  // offsets and tile prefixes: lane l owns experts l*VPL .. l*VPL+VPL-1
  if (wv == 0) {
    int c[VPL], s_rows = 0, s_t64 = 0, s_t256 = 0;
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      const int e = lane * VPL + v;
      c[v] = e < E ? cnt[e] : 0;
      s_rows += c[v];
      s_t64 += (c[v] + a.tile_m - 1) / a.tile_m;
      s_t256 += (c[v] + a.tile_m_big - 1) / a.tile_m_big;
    }
    int i_rows = s_rows, i_t64 = s_t64, i_t256 = s_t256;  // inclusive scans over lanes
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int r = __shfl_up(i_rows, o, 64), q = __shfl_up(i_t64, o, 64), u = __shfl_up(i_t256, o, 64);
      if (lane >= o) { i_rows += r; i_t64 += q; i_t256 += u; }
    }
    int o_rows = i_rows - s_rows, o_t64 = i_t64 - s_t64, o_t256 = i_t256 - s_t256;
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      const int e = lane * VPL + v;
      if (e < E) {
        off[e] = o_rows;
        tpb[e] = o_t256;
        a.offsets[e] = o_rows;
        if (a.user_offsets) a.user_offsets[e] = o_rows;
        a.tile_prefix[e] = o_t64;
        a.tile_prefix_big[e] = o_t256;
      }
      o_rows += c[v];
      o_t64 += (c[v] + a.tile_m - 1) / a.tile_m;
      o_t256 += (c[v] + a.tile_m_big - 1) / a.tile_m_big;
    }
    if (lane == 63) {  // totals: off[E] = P; the shared expert's T rows follow
      off[E] = o_rows;
      a.offsets[E] = o_rows;
      if (a.user_offsets) a.user_offsets[E] = o_rows;
      int t64 = o_t64, t256 = o_t256;
      tpb[E] = t256;
      if (a.shared) {
        a.offsets[E + 1] = o_rows + T;
        a.tile_prefix[E] = t64;
        a.tile_prefix_big[E] = t256;
        t64 += (T + a.tile_m - 1) / a.tile_m;
        t256 += (T + a.tile_m_big - 1) / a.tile_m_big;
        tpb[E + 1] = t256;
      }
      const int Eall = E + (a.shared ? 1 : 0);
      a.tile_prefix[Eall] = t64;
      a.tile_prefix_big[Eall] = t256;
    }
  }
  __syncthreads();

  // one descriptor per 256-row tile: {expert, first row, end row, 0}
  const int Eall = E + (a.shared ? 1 : 0);
  for (int e = tid; e < Eall; e += 1024) {
    const int first = tpb[e];
    const int n = tpb[e + 1] - first;
    const int r_begin = e < E ? off[e] : off[E];
    const int r_end = e < E ? off[e] + cnt[e] : off[E] + T;
    for (int j = 0; j < n; ++j) {
      int32_t* dsc = a.tile_desc + 4 * (size_t)(first + j);
      dsc[0] = e;
      dsc[1] = r_begin + j * a.tile_m_big;
      dsc[2] = r_end;
      dsc[3] = 0;
    }
  }
  // stable rank of pair p among the earlier pairs of its expert
  if (tid < P) {
    const int e = chosen[tid];
    int rank = 0;
    for (int q = 0; q < tid; ++q) rank += chosen[q] == e;
    const int dest = off[e] + rank;
    a.sorted_pair[dest] = tid;
    a.row_token[dest] = tid / k;
    a.pos[tid] = dest;
    if (a.user_sorted) a.user_sorted[dest] = tid;
  }
  if (a.shared && tid < T) {
    a.sorted_pair[P + tid] = -1;
    a.row_token[P + tid] = tid;
  }
}

}  // namespace

hipError_t launch_permute(const Layer& L, const Work& W, hipStream_t s) {
  PermuteArgs a;
  a.idx = W.idx; a.hist = W.hist;
  a.T = L.T; a.k = L.k; a.E = L.E;
  const int rb = route_block_tokens(L);
  a.n_hist = (L.T + rb - 1) / rb;
  a.hist_per_block = kPermuteTokens / rb;
  const int nblk = (L.T + kPermuteTokens - 1) / kPermuteTokens;
  a.shared = L.has_shared() ? 1 : 0;
  a.tile_m = kTileM;
  a.tile_m_big = kTileMBig;
  a.offsets = W.offsets; a.tile_prefix = W.tile_prefix; a.tile_prefix_big = W.tile_prefix_big;
  a.tile_desc = W.tile_desc;
  a.sorted_pair = W.sorted_pair; a.row_token = W.row_token; a.pos = W.pos;
  a.user_offsets = L.routing.expert_offsets; a.user_sorted = L.routing.sorted_pair;
  if (few_token_route(L)) {
    const RouteArgs ra = route_args(L, W);
    if (L.E <= 64) select_permute_small_kernel<1><<<1, 1024, 0, s>>>(ra, a, W.route_part);
    else if (L.E <= 128) select_permute_small_kernel<2><<<1, 1024, 0, s>>>(ra, a, W.route_part);
    else select_permute_small_kernel<4><<<1, 1024, 0, s>>>(ra, a, W.route_part);
    return hipGetLastError();
  }
  permute_kernel<<<nblk, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace moe
