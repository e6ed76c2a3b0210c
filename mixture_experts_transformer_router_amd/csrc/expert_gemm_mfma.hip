// Grouped expert GEMMs on bf16 MFMA (many tokens per expert).
//
//   gate|up:  for sorted row r of expert e with token t = row_token[r]
//             h[r][f] = act(x[t] . Wg[e][f] + bg[e][f], x[t] . Wu[e][f] + bu[e][f])
//   down:     y[r][n] = h[r] . Wd[e][n] + bd[e][n]
//
// (MaxText GPT-OSS weight mapping "MOE EXPERTS"; glm4_moe_lite.go
// SwitchMLP.Forward: per-expert gathered products, activation, down product;
// SharedExperts.Forward for the shared expert, handled as expert E.)
//
// Block tile 256 rows x (64 NJ) columns; K is staged BK at a time through NS
// LDS buffers.  Global -> LDS copies go straight into LDS (no registers) and
// run NS - 1 tiles ahead of the multiply, so the latency of a copy is covered
// by NS - 1 tiles of MFMA work.
// 4 wavefronts, each owning a 128 x (32 NJ) sub-tile as 4 x NJ results of
// v_mfma_f32_32x32x16_bf16 (fp32 accumulators).  An LDS row holds BK bf16;
// its 16-byte chunks are stored XOR-swizzled by the row's position within a
// 128-byte line group, so the 16-byte fragment reads of 8 consecutive rows
// hit 8 different bank groups.
//
// gate|up: the block's 256 columns are 128 gate and the same 128 up rows of
// the expert, interleaved by 32 (gate, up, gate, up within each wavefront), so
// one lane holds g and u of the same (row, f) and the activation is applied
// in registers.  Token rows are gathered while loading (no permuted copy of
// x).  MXFP4 weights: the loader decodes e2m1 codes with their e8m0 block
// scale to bf16 in LDS (exact: every value is a bf16 number).
#include <type_traits>

#include "device_common.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int BM = kTileMBig;  // 256
constexpr int kThreads = 256;
constexpr int kXcds = 8;       // MI355X: workgroup i runs on XCD i % 8
// Tuning knobs (compile-time; -D overrides for sweeps).
#ifndef MOE_GEMM_GROUP_M
#define MOE_GEMM_GROUP_M 4
#endif
#ifndef MOE_GEMM_BK
#define MOE_GEMM_BK 64
#endif
#ifndef MOE_GEMM_STAGES
#define MOE_GEMM_STAGES 2
#endif
#ifndef MOE_GEMM_COPY_VIA_REGS
#define MOE_GEMM_COPY_VIA_REGS 0
#endif
constexpr int kGroupM = MOE_GEMM_GROUP_M;  // row tiles walked together within an XCD
// 0: global -> LDS copies (global_load_lds); 1: global -> registers at the
// start of a tile, registers -> LDS after its last barrier.
constexpr bool kCopyViaRegs = MOE_GEMM_COPY_VIA_REGS != 0;
constexpr int kBK = MOE_GEMM_BK;           // K elements per LDS stage
constexpr int kStages = MOE_GEMM_STAGES;   // LDS stages (copies run this many tiles ahead)

typedef float f32x16_t __attribute__((ext_vector_type(16)));

// D (32 x 32) += A (32 x 16) * B (16 x 32).  Lane l supplies A row (l % 32),
// k = 8 (l / 32) .. +7, and B column (l % 32), the same k; it holds D column
// (l % 32), rows 8 j + 4 (l / 32) + i in register 4 j + i.
__device__ __forceinline__ f32x16_t mfma_32x32x16(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

struct MfmaArgs {
  const uint16_t* a;          // gate|up: x [T, lda]; down: h [rows, lda]
  int lda;
  const int32_t* row_token;   // gate|up: token of each sorted row; down: nullptr
  const uint16_t* w0;         // dense [E, N, K] (down, or gate)
  const uint16_t* w1;         // dense up
  const uint8_t* c0;          // MXFP4 codes [E, N, K/2] / scales [E, N, K/32]
  const uint8_t* s0;
  const uint8_t* c1;
  const uint8_t* s1;
  const uint16_t* bias0;      // [E, N] or nullptr
  const uint16_t* bias1;
  const uint16_t* sh_w0;      // shared expert [N_sh, K_sh] or nullptr
  const uint16_t* sh_w1;
  int N, K, N_sh, K_sh;
  int E, E_all;
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

// 8 e2m1 codes (one 32-bit word, element 0 in the low nibble) times the block
// scale 2^(s - 127) -> 8 bf16.
__device__ __forceinline__ u32x4_t decode_e2m1x8(uint32_t codes, uint32_t s) {
  // fp32 bit patterns of 0, 0.5, 1, 1.5, 2, 3, 4, 6
  constexpr uint32_t kMag[8] = {0x00000000u, 0x3f000000u, 0x3f800000u, 0x3fc00000u,
                                0x40000000u, 0x40400000u, 0x40800000u, 0x40c00000u};
  const float scale = s == 0 ? __uint_as_float(0x00400000u)
                             : (s == 255 ? __uint_as_float(0x7fc00000u) : __uint_as_float(s << 23));
  uint32_t h[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t c = (codes >> (4 * i)) & 15u;
    const float v = __uint_as_float(kMag[c & 7u] | ((c & 8u) << 28)) * scale;
    h[i] = __float_as_uint(v) >> 16;  // exact: the low 16 bits are zero
  }
  return u32x4_t{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
}

// NJ = 32-column result tiles per wavefront (block columns BN = 64 NJ).
// NJ = 32-column result tiles per wavefront (block columns BN = 64 NJ);
// BK = K elements per stage; NS = LDS stages.
template <int WF, bool GATED, int NJ, int BK, int NS>
__global__ __launch_bounds__(kThreads, 1) void mfma_gemm_kernel(MfmaArgs a) {
  constexpr int BN = 64 * NJ;
  constexpr int CPR = BK / 8;             // 16-byte chunks per LDS row
  constexpr int SEG_ROWS = 1024 / (2 * BK);  // rows per 1 KB copy segment
  constexpr int RA = BM * CPR / kThreads; // copy rounds per stage, A
  constexpr int RB = BN * CPR / kThreads; // copy rounds per stage, B (dense)
  constexpr int R = RA + (WF == WF_MXFP4 ? 0 : RB);
  static_assert(!GATED || NJ % 2 == 0, "gate|up pairs need an even number of column tiles");
  static_assert(NS >= 2 && NS <= 4, "LDS stages");
  constexpr bool REGS = kCopyViaRegs && WF != WF_MXFP4;  // MXFP4 B goes through registers anyway
  static_assert(BM * CPR % kThreads == 0 && BN * CPR % kThreads == 0, "copy rounds");
  __shared__ uint16_t lds[NS][2][BM * BK];  // [stage][A | B]

  // Tile order.  The real number of row tiles is known only on the device;
  // every block reads it and the blocks of XCD x take the x-th contiguous
  // share of the tiles, walked kGroupM row tiles at a time, so the blocks
  // resident on one XCD reuse each other's A and B tiles through its L2.
  const int total_m = a.tile_prefix[a.E_all];
  const int total = total_m * a.n_tiles;
  const int xcd = blockIdx.x % kXcds, j = blockIdx.x / kXcds;
  const int share = (total + kXcds - 1) / kXcds;
  const int L = xcd * share + j;
  if (j >= share || L >= total) return;
  const int group = L / (kGroupM * a.n_tiles);
  const int first_m = group * kGroupM;
  const int gm = min(kGroupM, total_m - first_m);
  const int rr = L - group * kGroupM * a.n_tiles;
  const int m_tile = first_m + rr % gm;
  const int n_tile = rr / gm;
  const int4 desc = reinterpret_cast<const int4*>(a.tile_desc)[m_tile];
  const int e = desc.x;
  const bool shared = e >= a.E;
  const int N = shared ? a.N_sh : a.N;
  const int K = shared ? a.K_sh : a.K;
  const int n0 = n_tile * (GATED ? BN / 2 : BN);
  if (n0 >= N) return;
  const int r0 = desc.y;
  const int r_end = desc.z;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv >> 1, wn = wv & 1;

  // ---- copy coordinates.  In round i, wavefront wv fills the 1 KB LDS
  // segment 4 i + wv: lane l writes 16-byte slot l, i.e. row
  // SEG_ROWS (4 i + wv) + l / CPR, stored chunk l % CPR, which holds the
  // logical chunk that swz() maps there.  Rows past the expert's last row (A)
  // or past N (B) copy a valid row instead: they only feed outputs that the
  // epilogue drops.
  const int ld_sub = lane / CPR;
  const int ld_phys = lane % CPR;
  // The hash of swz() depends on row bits 1..4 (BK 32) or 0..5 (BK 64);
  // segments start at multiples of SEG_ROWS (16 or 8 rows), so the hash of a
  // copied row also depends on its segment: computed per round below.
  int a_row[RA];
#pragma unroll
  for (int i = 0; i < RA; ++i) {
    const int r = SEG_ROWS * (4 * i + wv) + ld_sub;
    const int gr = r0 + r < r_end ? r0 + r : r0;
    a_row[i] = a.row_token ? a.row_token[gr] : gr;
  }
  int b_row[RB];
#pragma unroll
  for (int i = 0; i < RB; ++i) {
    const int r = SEG_ROWS * (4 * i + wv) + ld_sub;
    int wrow, up = 0;
    if constexpr (GATED) {
      const int q = r >> 6, sub = r & 63;
      wrow = n0 + 32 * q + (sub & 31);
      up = sub >= 32;
    } else {
      wrow = n0 + r;
    }
    if (wrow >= N) wrow = n0;
    b_row[i] = (wrow << 1) | up;
  }
  const uint16_t* w_gate = shared ? a.sh_w0 : a.w0 + (size_t)e * a.N * K;
  const uint16_t* w_up = GATED ? (shared ? a.sh_w1 : a.w1 + (size_t)e * a.N * K) : nullptr;

  // MXFP4: thread t < BN decodes B row t through registers
  const uint8_t* mx_codes = nullptr;
  const uint8_t* mx_scales = nullptr;
  if constexpr (WF == WF_MXFP4) {
    const int r = tid < BN ? tid : BN - 1;
    int wrow;
    bool up = false;
    if constexpr (GATED) {
      const int q = r >> 6, sub = r & 63;
      wrow = n0 + 32 * q + (sub & 31);
      up = sub >= 32;
    } else {
      wrow = n0 + r;
    }
    if (wrow < N) {
      const size_t row = (size_t)e * a.N + wrow;
      mx_codes = (up ? a.c1 : a.c0) + row * (K / 2);
      mx_scales = (up ? a.s1 : a.s0) + row * (K / 32);
    }
  }
  u32x4_t mxr[2];   // codes of BK elements (BK / 2 bytes)
  uint32_t mxs[2];  // their scale bytes (one per 32 elements)

  // Every tile issues exactly R copy instructions per wavefront (the K tail
  // copies clamped, valid addresses and is zeroed after it lands), so the
  // counted waits below are exact.
  // logical chunk that lane slot ld_phys of round i holds (inverse of swz)
  auto ld_chunk_of = [&](int i) {
    const int row = SEG_ROWS * (4 * i + wv) + ld_sub;
    return (swz<BK>(row, ld_phys) - row * BK) >> 3;  // XOR is an involution
  };
  u32x4_t stage_a[REGS ? RA : 1], stage_b[REGS ? RB : 1];
  // register path: fetch tile kt into registers
  auto fetch_regs = [&](int kt) {
    if constexpr (REGS) {
#pragma unroll
      for (int i = 0; i < RA; ++i) {
        const int k = min(kt * BK + 8 * ld_chunk_of(i), K - 8);
        stage_a[i] = *reinterpret_cast<const u32x4_t*>(a.a + (size_t)a_row[i] * a.lda + k);
      }
      if constexpr (WF != WF_MXFP4) {
#pragma unroll
        for (int i = 0; i < RB; ++i) {
          const int k = min(kt * BK + 8 * ld_chunk_of(i), K - 8);
          const uint16_t* wsrc = (b_row[i] & 1) ? w_up : w_gate;
          stage_b[i] = *reinterpret_cast<const u32x4_t*>(wsrc + (size_t)(b_row[i] >> 1) * K + k);
        }
      }
    }
  };
  // register path: store the fetched tile into its stage
  auto land_regs = [&](int kt) {
    if constexpr (REGS) {
      uint16_t* As = lds[kt % NS][0];
      uint16_t* Bs = lds[kt % NS][1];
#pragma unroll
      for (int i = 0; i < RA; ++i) *reinterpret_cast<u32x4_t*>(As + (4 * i + wv) * 512 + 8 * lane) = stage_a[i];
      if constexpr (WF != WF_MXFP4) {
#pragma unroll
        for (int i = 0; i < RB; ++i) *reinterpret_cast<u32x4_t*>(Bs + (4 * i + wv) * 512 + 8 * lane) = stage_b[i];
      }
    }
  };
  auto issue_tile = [&](int kt) {
    const int stage = kt % NS;
    uint16_t* As = lds[stage][0];
    uint16_t* Bs = lds[stage][1];
    if constexpr (REGS) {
      (void)As; (void)Bs;
      return;
    }
#pragma unroll
    for (int i = 0; i < RA; ++i) {
      const int k = min(kt * BK + 8 * ld_chunk_of(i), K - 8);
      __builtin_amdgcn_global_load_lds(a.a + (size_t)a_row[i] * a.lda + k, As + (4 * i + wv) * 512, 16, 0, 0);
    }
    if constexpr (WF == WF_MXFP4) {
      const int k0 = kt * BK;
#pragma unroll
      for (int h = 0; h < BK / 32; ++h) {
        const bool ok = mx_codes && k0 + 32 * h < K;
        mxr[h] = ok ? *reinterpret_cast<const u32x4_t*>(mx_codes + k0 / 2 + 16 * h) : u32x4_t{0u, 0u, 0u, 0u};
        mxs[h] = ok ? (uint32_t)mx_scales[k0 / 32 + h] : 127u;
      }
    } else {
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        const int k = min(kt * BK + 8 * ld_chunk_of(i), K - 8);
        const uint16_t* wsrc = (b_row[i] & 1) ? w_up : w_gate;
        __builtin_amdgcn_global_load_lds(wsrc + (size_t)(b_row[i] >> 1) * K + k, Bs + (4 * i + wv) * 512, 16, 0, 0);
      }
    }
  };
  // MXFP4 only: decode the staged codes of row tid into the tile's stage
  auto finish_tile = [&](int kt) {
    if constexpr (WF == WF_MXFP4) {
      uint16_t* Bs = lds[kt % NS][1];
      if (tid < BN) {
#pragma unroll
        for (int c = 0; c < CPR; ++c)
          *reinterpret_cast<u32x4_t*>(Bs + swz<BK>(tid, c)) = decode_e2m1x8(mxr[c / 4][c % 4], mxs[c / 4]);
      }
    }
  };
  // zero the chunks of the tile past K (the last tile only)
  auto zero_tail = [&](int kt) {
    uint16_t* As = lds[kt % NS][0];
    uint16_t* Bs = lds[kt % NS][1];
#pragma unroll
    for (int i = 0; i < RA; ++i)
      if (kt * BK + 8 * ld_chunk_of(i) >= K)
        *reinterpret_cast<u32x4_t*>(As + (4 * i + wv) * 512 + 8 * lane) = u32x4_t{0u, 0u, 0u, 0u};
    if constexpr (WF != WF_MXFP4) {
#pragma unroll
      for (int i = 0; i < RB; ++i)
        if (kt * BK + 8 * ld_chunk_of(i) >= K)
          *reinterpret_cast<u32x4_t*>(Bs + (4 * i + wv) * 512 + 8 * lane) = u32x4_t{0u, 0u, 0u, 0u};
    }
  };

  f32x16_t acc[4][NJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  // ---- pipeline.  The copies of tile t are issued NS tiles ahead: the
  // prologue issues tiles 0 .. NS-1 into all stages; in the last 16-wide K
  // step of tile kt the block waits for tile kt+1, meets at a barrier (after
  // which nobody reads tile kt from LDS: its last fragments are in
  // registers), issues tile kt+NS into tile kt's stage and reads the first
  // fragments of tile kt+1, all before the last MFMAs of tile kt.  Within a
  // tile the fragments of step kk+1 are read while step kk multiplies (two
  // register sets).  sched_barrier(0) keeps the compiler from sinking those
  // reads below the MFMAs they are meant to overlap.
  constexpr int KK = BK / 16;
  static_assert(KK % 2 == 0, "fragment double buffering needs an even step count");
  const int ktiles = (K + BK - 1) / BK;
  const int tail_tile = (K % BK) != 0 ? ktiles - 1 : -1;
  const int fr = lane & 31, fk = lane >> 5;

  bf16x8_t fa[2][4], fb[2][NJ];
  auto load_frags = [&](int stage, int kk, int buf) {
    const uint16_t* As = lds[stage][0];
    const uint16_t* Bs = lds[stage][1];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      fa[buf][i] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(As + swz<BK>(wm * 128 + 32 * i + fr, 2 * kk + fk)));
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      fb[buf][j] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(Bs + swz<BK>(wn * 32 * NJ + 32 * j + fr, 2 * kk + fk)));
  };
  // wait until tile t has landed, given that tiles up to `last` are issued
  auto wait_tile = [&](int t, int last) {
    const int after = last - t;  // tiles issued after t
    if constexpr (WF == WF_MXFP4) {
      wait_vmcnt<0>();
    } else {
      if (NS >= 4 && after >= 3) wait_vmcnt<(NS >= 4 ? 3 * R : 0)>();
      else if (NS >= 3 && after >= 2) wait_vmcnt<(NS >= 3 ? 2 * R : 0)>();
      else if (NS >= 2 && after >= 1) wait_vmcnt<(NS >= 2 ? R : 0)>();
      else wait_vmcnt<0>();
    }
  };

#pragma unroll
  for (int t = 0; t < NS; ++t) {
    if (t < ktiles) {
      issue_tile(t);
      finish_tile(t);
      fetch_regs(t);
      land_regs(t);
    }
  }
  if constexpr (REGS) wait_vmcnt<0>();
  else wait_tile(0, min(NS - 1, ktiles - 1));
  barrier_lds();
  if (tail_tile == 0) {
    zero_tail(0);
    barrier_lds();
  }
  load_frags(0, 0, 0);
  // One K tile.  STEADY: tiles kt+1 and kt+NS exist and kt+1 is no tail, so
  // the step runs without branches (and the compiler's wait counting stays exact).
  auto tile_step = [&](int kt, auto steady_tag) {
    constexpr bool STEADY = decltype(steady_tag)::value;
    const int st = kt % NS;
    if (REGS && (STEADY || kt + NS < ktiles)) fetch_regs(kt + NS);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const int cur = kk & 1;
      if (kk + 1 < KK) {
        // this step's fragments were read a whole MFMA run ago; waiting for
        // them here keeps the wait from also covering the reads issued next
        wait_lgkmcnt0();
        load_frags(st, kk + 1, cur ^ 1);
      } else if (STEADY || kt + 1 < ktiles) {
        if constexpr (REGS) wait_vmcnt<0>();  // the registers of tile kt+NS
        else if (STEADY) wait_tile(kt + 1, kt + NS - 1);
        else wait_tile(kt + 1, min(kt + NS - 1, ktiles - 1));
        barrier_lds();  // tile kt+1 is in LDS; every wavefront is done reading tile kt
        if (!STEADY && kt + 1 == tail_tile) {
          zero_tail(kt + 1);
          barrier_lds();
        }
        if (STEADY || kt + NS < ktiles) {
          issue_tile(kt + NS);
          land_regs(kt + NS);
        }
        load_frags((kt + 1) % NS, 0, cur ^ 1);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = mfma_32x32x16(fa[cur][i], fb[cur][j], acc[i][j]);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (STEADY || kt + NS < ktiles) finish_tile(kt + NS);
  };
  int kt = 0;
  // steady state needs tile kt+NS < ktiles and no tail tile at kt+1
  const int steady_end = ktiles - NS - (tail_tile >= 0 ? 1 : 0);
  for (; kt < steady_end; ++kt) tile_step(kt, std::true_type{});
  for (; kt < ktiles; ++kt) tile_step(kt, std::false_type{});
  wait_vmcnt<0>();
  barrier_lds();  // every wavefront is done with the stages before they are reused

  // ---- epilogue.  Bias (+ activation) in registers.  A lane holds one
  // column for 16 rows of each 32 x 32 result; a 4 x 4 transpose across each
  // lane quad (two xor shuffles) gives it 4 consecutive columns of one row,
  // stored as 8 bytes straight to HBM (8 lanes write a 64-byte row piece).
  const uint16_t* bias0 = shared ? nullptr : a.bias0;
  const uint16_t* bias1 = shared ? nullptr : a.bias1;
  const int act = shared ? 1 : a.act;
  const int c4 = fr & 3;            // position in the lane quad
  constexpr int OJ = GATED ? NJ / 2 : NJ;  // output column tiles per wavefront
  float bv0[OJ], bv1[OJ];
  int colj[OJ];
#pragma unroll
  for (int j = 0; j < OJ; ++j) {
    colj[j] = GATED ? n0 + 32 * (2 * wn + j) : n0 + wn * 32 * NJ + 32 * j;
    const int c = colj[j] + fr;
    bv0[j] = (bias0 && c < N) ? bf16_to_f32(bias0[(size_t)e * N + c]) : 0.f;
    bv1[j] = (GATED && bias1 && c < N) ? bf16_to_f32(bias1[(size_t)e * N + c]) : 0.f;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {      // groups of 4 consecutive rows (q = 4 g .. 4 g + 3)
      const int row_base = wm * 128 + 32 * i + 8 * g + 4 * fk;
#pragma unroll
      for (int j = 0; j < OJ; ++j) {
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int q = 4 * g + r;
          if constexpr (GATED) v[r] = expert_act(act, acc[i][2 * j][q] + bv0[j], acc[i][2 * j + 1][q] + bv1[j], a.alpha, a.limit);
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
        const int row = r0 + row_base + c4;
        const int col = colj[j] + (fr & ~3);
        if (row < r_end && col < N) {
          *reinterpret_cast<uint2*>(a.out + (size_t)row * a.ldo + col) =
              make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        }
      }
    }
  }
}

MfmaArgs base_args(const Layer& L, const Work& W) {
  MfmaArgs m{};
  m.E = L.E;
  m.E_all = L.n_experts_all();
  m.offsets = W.offsets;
  m.tile_prefix = W.tile_prefix_big;
  m.tile_desc = W.tile_desc;
  m.act = L.act;
  m.alpha = L.alpha;
  m.limit = L.limit;
  return m;
}

int max_row_tiles(const Layer& L) { return (L.rows_all() + BM - 1) / BM + L.n_experts_all(); }
int grid_for(int tiles) { return (tiles + kXcds - 1) / kXcds * kXcds; }

}  // namespace

hipError_t launch_gate_up_mfma(const Layer& L, const Work& W, hipStream_t s) {
  MfmaArgs m = base_args(L, W);
  m.a = static_cast<const uint16_t*>(L.x);
  m.lda = L.d;
  m.row_token = W.row_token;
  m.w0 = static_cast<const uint16_t*>(L.wg);
  m.w1 = static_cast<const uint16_t*>(L.wu);
  m.c0 = L.wg_codes; m.s0 = L.wg_scales; m.c1 = L.wu_codes; m.s1 = L.wu_scales;
  m.bias0 = static_cast<const uint16_t*>(L.bg);
  m.bias1 = static_cast<const uint16_t*>(L.bu);
  m.sh_w0 = static_cast<const uint16_t*>(L.sh_wg);
  m.sh_w1 = static_cast<const uint16_t*>(L.sh_wu);
  m.N = L.F; m.K = L.d; m.N_sh = L.F_sh; m.K_sh = L.d;
  m.out = static_cast<uint16_t*>(W.h);
  m.ldo = L.F_max();
  m.n_tiles = (L.F_max() + 127) / 128;
  const dim3 grid(grid_for(max_row_tiles(L) * m.n_tiles));
  if (L.wfmt == WF_MXFP4) mfma_gemm_kernel<WF_MXFP4, true, 4, kBK, kStages><<<grid, kThreads, 0, s>>>(m);
  else mfma_gemm_kernel<WF_BF16, true, 4, kBK, kStages><<<grid, kThreads, 0, s>>>(m);
  return hipGetLastError();
}

hipError_t launch_down_mfma(const Layer& L, const Work& W, hipStream_t s) {
  MfmaArgs m = base_args(L, W);
  m.a = static_cast<const uint16_t*>(W.h);
  m.lda = L.F_max();
  m.row_token = nullptr;
  m.w0 = static_cast<const uint16_t*>(L.wd);
  m.c0 = L.wd_codes; m.s0 = L.wd_scales;
  m.bias0 = static_cast<const uint16_t*>(L.bd);
  m.sh_w0 = static_cast<const uint16_t*>(L.sh_wd);
  m.N = L.d; m.K = L.F; m.N_sh = L.d; m.K_sh = L.F_sh;
  m.out = static_cast<uint16_t*>(W.y);
  m.ldo = L.d;
  // 192-column tiles when they waste fewer columns than 256-column ones
  const int t192 = (L.d + 191) / 192, t256 = (L.d + 255) / 256;
  const bool narrow = t192 * 192 < t256 * 256;
  m.n_tiles = narrow ? t192 : t256;
  const dim3 grid(grid_for(max_row_tiles(L) * m.n_tiles));
  if (L.wfmt == WF_MXFP4) {
    if (narrow) mfma_gemm_kernel<WF_MXFP4, false, 3, kBK, kStages><<<grid, kThreads, 0, s>>>(m);
    else mfma_gemm_kernel<WF_MXFP4, false, 4, kBK, kStages><<<grid, kThreads, 0, s>>>(m);
  } else {
    if (narrow) mfma_gemm_kernel<WF_BF16, false, 3, kBK, kStages><<<grid, kThreads, 0, s>>>(m);
    else mfma_gemm_kernel<WF_BF16, false, 4, kBK, kStages><<<grid, kThreads, 0, s>>>(m);
  }
  return hipGetLastError();
}

}  // namespace moe
