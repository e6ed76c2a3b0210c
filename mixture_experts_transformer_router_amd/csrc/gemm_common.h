// Pieces shared by the grouped expert GEMMs on bf16 MFMA (dense bf16 and
// MXFP4 weights): the 256-row tile geometry, the XCD-aware tile order, LDS
// swizzle, pipeline waits, the activation, and the bias/activation epilogue.
#pragma once

#include "device_common.h"
#include "moe_internal.h"

namespace moe {
namespace gemm {

constexpr int BM = kTileMBig;  // 256
constexpr int kThreads = 256;
constexpr int kXcds = 8;       // MI355X: workgroup i runs on XCD i % 8

typedef float f32x16_t __attribute__((ext_vector_type(16)));

// D (32 x 32) += A (32 x 16) * B (16 x 32).  Lane l supplies A row (l % 32),
// k = 8 (l / 32) .. +7, and B column (l % 32), the same k; it holds D column
// (l % 32), rows 8 j + 4 (l / 32) + i in register 4 j + i.
__device__ __forceinline__ f32x16_t mfma_32x32x16(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

struct MfmaArgs {
  const uint16_t* a;          // gate|up: x [T, lda]; down: h [rows, lda] (MXFP8: E4M3 codes, lda bytes a row)
  int lda;
  const int32_t* row_token;   // gate|up: token of each sorted row; down: nullptr
  int a_row0;                 // without row_token: A row of sorted row r is r - a_row0
  const uint16_t* zrow;       // zeros (at least K of them) for the A rows past a tile's last row, or
                              // nullptr (those rows then copy the tile's first row)
  const uint16_t* w0;         // dense [E, N, K] (down, or gate)
  const uint16_t* w1;         // dense up
  const uint8_t* c0;          // low-bit codes [E, N, K * bits / 8]; scales: MXFP4 e8m0 bytes
  const uint8_t* s0;          // [E, N, K / 32], affine bf16 [E, N, K / group]
  const uint8_t* c1;
  const uint8_t* s1;
  const uint8_t* as;          // MXFP8 activations: e8m0 scales [rows, lda / 32] of the codes at a
  const uint16_t* qb0;        // affine: bf16 biases [E, N, K / group] of c0 / c1
  const uint16_t* qb1;
  float ts0, ts1;             // NVFP4: tensor scales of c0 / c1
  const uint16_t* bias0;      // [E, N] or nullptr
  const uint16_t* bias1;
  const uint16_t* sh_w0;      // shared expert [N_sh, K_sh] or nullptr
  const uint16_t* sh_w1;
  int N, K, N_sh, K_sh;
  int E, E_all;
  int e_first, e_end;         // the launch covers the tiles of experts [e_first, e_end)
  const int32_t* offsets;     // [E_all + 1]
  const int32_t* tile_prefix; // [E_all + 1], 256-row tiles
  const int32_t* tile_desc;   // [tiles][4]: expert, first row, end row
  int n_tiles;                // column tiles per row tile
  uint16_t* out;
  int ldo;
  int act;
  float alpha, limit;
};

// Element offset of 16-byte chunk `chunk` of LDS row `row` (rows of BK bf16).
// The chunk is XOR-ed with a row hash chosen so that the 16-byte reads of
// any 8 consecutive rows (same logical chunk) fall in 8 distinct 16-byte
// slots of a 128-byte bank window, and those of any 16 consecutive rows
// (32-aligned groups, as the fragment reads use) in 16 distinct slots of a
// 256-byte window: conflict-free whether the LDS serves 8 or 16 lanes of a
// 16-byte read per clock.
template <int BK>
__device__ __forceinline__ int swz(int row, int chunk) {
  constexpr int CPR = BK / 8;  // chunks per row: 4 (BK 32) or 8 (BK 64)
  int h;
  if constexpr (CPR == 4) h = ((row >> 1) ^ (row >> 3)) & 3;
  else h = (row ^ (row >> 3)) & 7;
  return row * BK + ((chunk ^ h) << 3);
}

// Workgroup barrier for the copy pipeline.  __syncthreads() would also drain
// every outstanding global -> LDS copy (its release fence covers them), which
// would serialise the pipeline; here each wavefront first waits for its own
// LDS stores and for the copies it needs (wait_vmcnt), then meets the others.
// The asm's memory clobber keeps the compiler from moving LDS accesses across.
__device__ __forceinline__ void barrier_lds() {
  // the wait is a builtin so that the compiler's own wait counting sees it
  __builtin_amdgcn_s_waitcnt((15 << 14) | 15 | (7 << 4));  // lgkmcnt(0)
  asm volatile("s_barrier" ::: "memory");
}

// Wait for this wavefront's outstanding LDS operations only (vmcnt and
// expcnt at their maxima).
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt((15 << 14) | 15 | (7 << 4)); }

// Wait until at most n vector-memory operations of this wavefront are
// outstanding (gfx9 s_waitcnt: vmcnt in bits 3:0 and 15:14; expcnt and
// lgkmcnt left at their maxima).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Value of lane l ^ 1 / l ^ 2 within each lane quad (DPP quad_perm [1,0,3,2] / [2,3,0,1]).
__device__ __forceinline__ float quad_xor1(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true));
}
__device__ __forceinline__ float quad_xor2(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true));
}

// The expert activation with its kind fixed at compile time (no per-element
// branch); the clamps keep NaN (clip_nan; the C ABI guarantees limit > 0).
// act 0: clipped SwiGLU, act 1: SiLU-GLU, as expert_act().
template <int ACT>
__device__ __forceinline__ float expert_act_t(float g, float u, float alpha, float limit) {
  if constexpr (ACT == 0) {
    const float gc = clip_nan(g, 0.f, limit);
    const float uc = clip_nan(u, -limit, limit);
    return gc * sigmoidf_(alpha * gc) * uc;
  } else {
    return g * sigmoidf_(g) * u;
  }
}

// Tile of this block.  The real number of row tiles is known only on the
// device; every block reads the row-tile prefix of its launch's experts
// [e_first, e_end) and the blocks of XCD x take the x-th contiguous share of
// the launch's tiles.  The tile list runs expert by expert (an expert's
// row tiles times the column tiles are contiguous in it); inside an expert it
// is walked kGroupM row tiles at a time, the column tile outermost, so the
// blocks resident on one XCD at a time cover a few row tiles of ONE expert
// times several column tiles and reuse each other's A rows and weight panels
// through that XCD's L2 (a group never mixes two experts' weights).  Returns
// false for blocks without a tile.
template <int kGroupM>
__device__ __forceinline__ bool block_tile(const MfmaArgs& a, int& m_tile, int& n_tile) {
  const int m_lo = a.tile_prefix[a.e_first];
  const int total_m = a.tile_prefix[a.e_end] - m_lo;
  const int nt = a.n_tiles;
  const int total = total_m * nt;
  const int xcd = blockIdx.x % kXcds, j = blockIdx.x / kXcds;
  const int share = (total + kXcds - 1) / kXcds;
  const int L = xcd * share + j;
  if (j >= share || L >= total) return false;
  // the expert whose tiles hold L: the last e with tile_prefix[e] * nt <= m_lo * nt + L
  int lo = a.e_first, hi = a.e_end;  // tile_prefix[lo] - m_lo <= L / nt < tile_prefix[hi] - m_lo
  const int mL = L / nt;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.tile_prefix[mid] - m_lo <= mL) lo = mid;
    else hi = mid;
  }
  const int e_m0 = a.tile_prefix[lo] - m_lo;              // first row tile of the expert (launch-relative)
  const int e_mt = a.tile_prefix[lo + 1] - m_lo - e_m0;   // its row tiles
  const int l = L - e_m0 * nt;                            // index inside the expert's tiles
  const int group = l / (kGroupM * nt);
  const int first_m = group * kGroupM;
  const int gm = min(kGroupM, e_mt - first_m);
  const int rr = l - group * kGroupM * nt;
  m_tile = m_lo + e_m0 + first_m + rr % gm;
  n_tile = rr / gm;
  return true;
}

// Epilogue of a 256 x (32 NJ WN) tile held by 2 x WN wavefronts (each
// 128 x 32 NJ as 4 x NJ results of 32 x 32): bias (+ activation) and bf16
// stores.
template <bool GATED, int NJ, int WN = 2>
__device__ __forceinline__ void store_tile(const MfmaArgs& a, f32x16_t (&acc)[4][NJ], int e, bool shared, int N,
                                           int n0, int r0, int r_end, int wm, int wn, int lane) {
  constexpr int BN = 32 * NJ * WN;
  const int fr = lane & 31, fk = lane >> 5;
  // A lane holds one column for 16 rows of each 32 x 32 result; a 4 x 4
  // transpose across each lane quad (two xor shuffles) gives it 4 consecutive
  // columns of one row, stored as 8 bytes straight to HBM (8 lanes write a
  // 64-byte row piece).
  const uint16_t* bias0 = shared ? nullptr : a.bias0;
  const uint16_t* bias1 = shared ? nullptr : a.bias1;
  const int act = shared ? 1 : a.act;
  const int c4 = fr & 3;            // position in the lane quad
  constexpr int OJ = GATED ? NJ / 2 : NJ;  // output column tiles per wavefront
  // this lane's first output row, and whether the whole tile is inside the
  // expert's rows and the N columns (then the stores need no bounds check)
  const int lane_row = r0 + wm * 128 + 4 * fk + c4;
  uint16_t* const lane_out = a.out + (size_t)lane_row * a.ldo + (fr & ~3);
  const bool tile_inside = r0 + BM <= r_end && n0 + (GATED ? BN / 2 : BN) <= N;
  float bv0[OJ], bv1[OJ];
  int colj[OJ];
#pragma unroll
  for (int j = 0; j < OJ; ++j) {
    colj[j] = GATED ? n0 + 32 * (OJ * wn + j) : n0 + wn * 32 * NJ + 32 * j;
    const int c = colj[j] + fr;
    bv0[j] = (bias0 && c < N) ? bf16_to_f32(bias0[(size_t)e * N + c]) : 0.f;
    bv1[j] = (GATED && bias1 && c < N) ? bf16_to_f32(bias1[(size_t)e * N + c]) : 0.f;
  }
  // the activation is a template argument of the loops (one copy per kind)
  auto epilogue = [&](auto act_tag, auto inside_tag) __attribute__((always_inline)) {
    constexpr int ACT = decltype(act_tag)::value;
    constexpr bool INSIDE = decltype(inside_tag)::value;  // no bounds checks
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {      // groups of 4 consecutive rows (q = 4 g .. 4 g + 3)
#pragma unroll
        for (int j = 0; j < OJ; ++j) {
          float v[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int q = 4 * g + r;
            if constexpr (GATED) v[r] = expert_act_t<ACT>(acc[i][2 * j][q] + bv0[j], acc[i][2 * j + 1][q] + bv1[j], a.alpha, a.limit);
            else v[r] = acc[i][j][q] + bv0[j];
          }
          // transpose within the lane quad: afterwards lane c4 holds row
          // row_base + c4, columns (fr & ~3) .. +3
          {
            const bool odd = c4 & 1;
            const float s0 = odd ? v[0] : v[1], s1 = odd ? v[2] : v[3];
            const float r0_ = quad_xor1(s0), r1_ = quad_xor1(s1);
            if (odd) { v[0] = r0_; v[2] = r1_; } else { v[1] = r0_; v[3] = r1_; }
            // lane even: v = [row 0 c, row 0 c+1, row 2 c, row 2 c+1]; odd: rows 1 and 3
          }
          {
            const bool hi = c4 & 2;
            const float s0 = hi ? v[0] : v[2], s1 = hi ? v[1] : v[3];
            const float r0_ = quad_xor2(s0), r1_ = quad_xor2(s1);
            if (hi) { v[0] = r0_; v[1] = r1_; } else { v[2] = r0_; v[3] = r1_; }
          }
          const int drow = 32 * i + 8 * g;  // row_base + c4 - (lane_row - r0)
          const int col = colj[j] + (fr & ~3);
          if (INSIDE || (lane_row + drow < r_end && col < N)) {
            *reinterpret_cast<uint2*>(lane_out + (size_t)drow * a.ldo + colj[j]) =
                make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
          }
        }
      }
    }
  };
  if (tile_inside) {
    if (!GATED || act == 0) epilogue(std::integral_constant<int, 0>{}, std::true_type{});
    else epilogue(std::integral_constant<int, 1>{}, std::true_type{});
  } else {
    if (!GATED || act == 0) epilogue(std::integral_constant<int, 0>{}, std::false_type{});
    else epilogue(std::integral_constant<int, 1>{}, std::false_type{});
  }
}

inline MfmaArgs base_args(const Layer& L, const Work& W) {
  MfmaArgs m{};
  m.E = L.E;
  m.E_all = L.n_experts_all();
  m.e_first = 0;
  m.e_end = m.E_all;
  m.offsets = W.offsets;
  m.tile_prefix = W.tile_prefix_big;
  m.tile_desc = W.tile_desc;
  m.act = L.act;
  m.alpha = L.alpha;
  m.limit = L.limit;
  m.zrow = nullptr;
  return m;
}

inline int max_row_tiles(const Layer& L) { return (L.rows_all() + BM - 1) / BM + L.n_experts_all(); }
// Bound on the row tiles of experts [e_first, e_end): the routed experts hold
// T k rows, the shared expert (index E) T rows, and each expert pads at most
// one tile.
inline int max_row_tiles(const Layer& L, int e_first, int e_end) {
  long long rows = 0;
  if (e_first < L.E) rows += (long long)L.T * L.k;
  if (e_end > L.E) rows += L.T;
  return (int)((rows + BM - 1) / BM) + (e_end - e_first);
}
inline int grid_for(int tiles) { return (tiles + kXcds - 1) / kXcds * kXcds; }

}  // namespace gemm
}  // namespace moe
