// The permutation block (one per kPermuteTokens tokens) as a device function
// of the block's index, with its arguments, so that the permutation's launch
// and a launch that also carries other work run the same code.  Included by
// permute.hip and expert_gemm_mfma.hip (device code of one translation unit
// each).
#pragma once

#include "route_common.h"

namespace moe {
namespace {

constexpr int kPermuteThreads = 256;
constexpr int kMaxE = 257;  // 256 routed experts + shared
constexpr int kScanPerLane = (kMaxE + 63) / 64;  // experts per lane in the offset scan

struct PermuteArgs {
  const int32_t* idx;
  const int32_t* hist;  // [n_hist, E] expert counts per router block
  int n_hist;           // router blocks
  int hist_per_block;   // router blocks per permute block (64 / router block tokens)
  int T, k, E, shared;
  int32_t* offsets;
  int32_t* tile_prefix;
  int32_t* tile_prefix_big;
  int32_t* tile_desc;
  int32_t* sorted_pair;
  int32_t* row_token;
  int32_t* pos;
  int32_t* user_offsets;
  int32_t* user_sorted;
  uint32_t* zrow;  // block 0 writes zrow_words zeros (the GEMMs' zero row), or nullptr
  int zrow_words;
};

__device__ __forceinline__ void permute_block(const PermuteArgs& a, int b) {
  __shared__ int total[kMaxE];
  __shared__ int before[kMaxE];
  __shared__ int off[kMaxE + 1];
  __shared__ int running[kMaxE];
  __shared__ int wcnt[4][kMaxE];
  __shared__ int tpb[kMaxE + 1];  // 256-row tile prefix (block 0)

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int E = a.E;
  if (b == 0 && a.zrow)
    for (int i = tid; i < a.zrow_words; i += kPermuteThreads) a.zrow[i] = 0u;

  // Column sums of the count table, split over all threads: thread
  // (part, e) adds rows part, part + parts, ... of expert e.
  {
    int* part_tot = &wcnt[0][0];           // scratch, cleared again below
    int* part_bef = &wcnt[2][0];
    const int parts = E >= kPermuteThreads ? 1 : kPermuteThreads / E;
    const int first_own = b * a.hist_per_block;
    for (int t = tid; t < parts * E; t += kPermuteThreads) {
      const int e = t % E, part = t / E;
      int tot = 0, bef = 0;
#pragma unroll 16
      for (int i = part; i < a.n_hist; i += parts) {
        const int c = a.hist[(size_t)i * E + e];
        tot += c;
        bef += i < first_own ? c : 0;
      }
      part_tot[t] = tot;
      part_bef[t] = bef;
    }
    __syncthreads();
    for (int e = tid; e < E; e += kPermuteThreads) {
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
  for (int i = tid; i < 4 * kMaxE; i += kPermuteThreads) (&wcnt[0][0])[i] = 0;
  // Exclusive scans of the expert counts (off: routed experts, off[E] = all
  // routed rows) and of their 64- and 256-row tile counts (tile prefixes:
  // the shared expert, if any, is expert E with T rows).  Wavefront 0, lane l
  // owning experts kScanPerLane l .. +kScanPerLane-1, a shuffle scan over the
  // lanes.  Block 0 also writes them out.
  const int Eall = E + (a.shared ? 1 : 0);
  if (wv == 0) {
    int rows[kScanPerLane], tiles[kScanPerLane];
    int s_rows = 0, s_t64 = 0, s_t256 = 0;
#pragma unroll
    for (int v = 0; v < kScanPerLane; ++v) {
      const int e = lane * kScanPerLane + v;
      rows[v] = e < E ? total[e] : 0;
      tiles[v] = e < E ? total[e] : e == E && a.shared ? a.T : 0;
      s_rows += rows[v];
      s_t64 += (tiles[v] + kTileM - 1) / kTileM;
      s_t256 += (tiles[v] + kTileMBig - 1) / kTileMBig;
    }
    int i_rows = s_rows, i_t64 = s_t64, i_t256 = s_t256;  // inclusive scans over lanes
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int r = __shfl_up(i_rows, o, 64), q = __shfl_up(i_t64, o, 64), u = __shfl_up(i_t256, o, 64);
      if (lane >= o) { i_rows += r; i_t64 += q; i_t256 += u; }
    }
    int o_rows = i_rows - s_rows, o_t64 = i_t64 - s_t64, o_t256 = i_t256 - s_t256;
#pragma unroll
    for (int v = 0; v < kScanPerLane; ++v) {
      const int e = lane * kScanPerLane + v;
      if (e <= E) off[e] = o_rows;
      if (e <= Eall) tpb[e] = o_t256;
      if (b == 0) {
        if (e <= E) {
          a.offsets[e] = o_rows;
          if (a.user_offsets) a.user_offsets[e] = o_rows;
        }
        if (e == E && a.shared) a.offsets[E + 1] = o_rows + a.T;
        if (e <= Eall) {
          a.tile_prefix[e] = o_t64;
          a.tile_prefix_big[e] = o_t256;
        }
      }
      o_rows += rows[v];
      o_t64 += (tiles[v] + kTileM - 1) / kTileM;
      o_t256 += (tiles[v] + kTileMBig - 1) / kTileMBig;
    }
  }
  __syncthreads();

  if (b == 0) {
    // one descriptor per 256-row tile: {expert, first row, end row, 0}
    for (int e = tid; e < Eall; e += kPermuteThreads) {
      const int first = tpb[e];
      const int n = tpb[e + 1] - first;
      const int r_begin = e < E ? off[e] : off[E];
      const int r_end = e < E ? off[e + 1] : off[E] + a.T;
      for (int j = 0; j < n; ++j) {
        int32_t* d = a.tile_desc + 4 * (size_t)(first + j);
        d[0] = e;
        d[1] = r_begin + j * kTileMBig;
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

  for (int r0 = 0; r0 < n; r0 += kPermuteThreads) {
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
    for (int ee = tid; ee < E; ee += kPermuteThreads) {
      running[ee] += wcnt[0][ee] + wcnt[1][ee] + wcnt[2][ee] + wcnt[3][ee];
      wcnt[0][ee] = wcnt[1][ee] = wcnt[2][ee] = wcnt[3][ee] = 0;
    }
    __syncthreads();
  }

  if (a.shared) {
    const int P = a.T * a.k;
    for (int t = t_begin + tid; t < t_end; t += kPermuteThreads) {
      a.sorted_pair[P + t] = -1;
      a.row_token[P + t] = t;
    }
  }
}

inline PermuteArgs permute_args(const Layer& L, const Work& W) {
  PermuteArgs a;
  a.idx = W.idx; a.hist = W.hist;
  a.T = L.T; a.k = L.k; a.E = L.E;
  const int rb = route_block_tokens(L);
  a.n_hist = (L.T + rb - 1) / rb;
  a.hist_per_block = kPermuteTokens / rb;
  a.shared = L.has_shared() ? 1 : 0;
  a.offsets = W.offsets; a.tile_prefix = W.tile_prefix; a.tile_prefix_big = W.tile_prefix_big;
  a.tile_desc = W.tile_desc;
  a.sorted_pair = W.sorted_pair; a.row_token = W.row_token; a.pos = W.pos;
  a.user_offsets = L.routing.expert_offsets; a.user_sorted = L.routing.sorted_pair;
  a.zrow = static_cast<uint32_t*>(W.zrow);
  a.zrow_words = W.zrow ? (int)(zero_row_bytes(L) / 4) : 0;
  return a;
}

}  // namespace
}  // namespace moe
