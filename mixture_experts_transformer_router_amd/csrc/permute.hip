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
#include "permute_common.h"

namespace moe {
namespace {

__global__ __launch_bounds__(kPermuteThreads) void permute_kernel(PermuteArgs a) { permute_block(a, blockIdx.x); }

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
  if (a.zrow)
    for (int i = tid; i < a.zrow_words; i += 1024) a.zrow[i] = 0u;
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
      s_t64 += (c[v] + kTileM - 1) / kTileM;
      s_t256 += (c[v] + kTileMBig - 1) / kTileMBig;
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
      o_t64 += (c[v] + kTileM - 1) / kTileM;
      o_t256 += (c[v] + kTileMBig - 1) / kTileMBig;
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
        t64 += (T + kTileM - 1) / kTileM;
        t256 += (T + kTileMBig - 1) / kTileMBig;
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
      dsc[1] = r_begin + j * kTileMBig;
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
  const PermuteArgs a = permute_args(L, W);
  if (few_token_route(L)) {
    const RouteArgs ra = route_args(L, W);
    if (L.E <= 64) select_permute_small_kernel<1><<<1, 1024, 0, s>>>(ra, a, W.route_part);
    else if (L.E <= 128) select_permute_small_kernel<2><<<1, 1024, 0, s>>>(ra, a, W.route_part);
    else select_permute_small_kernel<4><<<1, 1024, 0, s>>>(ra, a, W.route_part);
    return hipGetLastError();
  }
  permute_kernel<<<(L.T + kPermuteTokens - 1) / kPermuteTokens, kPermuteThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace moe
