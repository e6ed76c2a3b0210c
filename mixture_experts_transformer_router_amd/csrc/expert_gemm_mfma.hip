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
// Block tile 256 rows x (64 NJ) columns; K is staged BK at a time through LDS
// buffers filled by global -> LDS copies (no registers).  The A operand (token
// rows: a few tens of megabytes, mostly cache hits) has NS buffers and runs
// NS - 1 tiles ahead of the multiply; the B operand (expert weights, streamed
// from HBM) may have NSB = NS + 1 buffers to run one tile further ahead.  On
// MI355X the copies are bound by the L2 requests a CU keeps in flight, not by
// how far ahead they are issued, so the default is NSB = NS = 2.
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
#ifndef MOE_GEMM_STAGES_B
#define MOE_GEMM_STAGES_B 2
#endif
constexpr int kGroupM = MOE_GEMM_GROUP_M;  // row tiles walked together within an XCD
constexpr int kBK = MOE_GEMM_BK;           // K elements per LDS stage
constexpr int kStages = MOE_GEMM_STAGES;   // LDS stages of the A operand
constexpr int kStagesB = MOE_GEMM_STAGES_B;  // LDS stages of the (dense) B operand
// MXFP4 weights: 64-wide stages (a thread decodes 32 code bytes per stage), 2 LDS stages
constexpr int kBKMx = 64;
constexpr int kStagesMx = 2;
#ifndef MOE_GEMM_INTERLEAVE
#define MOE_GEMM_INTERLEAVE 1
#endif
// 1: the copies issued at a tile boundary alternate with that step's MFMAs
// (instead of one burst ahead of them), so the address unit works through
// them while the matrix cores run.
constexpr bool kInterleave = MOE_GEMM_INTERLEAVE != 0;
#ifndef MOE_GEMM_INTERLEAVE_LDS
#define MOE_GEMM_INTERLEAVE_LDS 1
#endif
// Within a tile, the fragment reads for step kk+1 follow the MFMAs of step
// kk one by one (1: after each of the first 4 + NJ MFMAs; 2: after every
// other MFMA) instead of coming as one burst ahead of them (0).
constexpr int kInterleaveLds = MOE_GEMM_INTERLEAVE_LDS;
#ifndef MOE_GEMM_BOUNDARY_READS
#define MOE_GEMM_BOUNDARY_READS 1
#endif
// At a tile boundary the first fragments of the next tile are read as one
// burst right after the barrier (0) or one after each MFMA/copy pair (1).
constexpr bool kBoundaryReadsInterleaved = MOE_GEMM_BOUNDARY_READS != 0;

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

// The expert activation with its kind fixed at compile time (no per-element
// branch); the clamps are single v_med3_f32 (the C ABI guarantees limit > 0).
// act 0: clipped SwiGLU, act 1: SiLU-GLU, as expert_act().
template <int ACT>
__device__ __forceinline__ float expert_act_t(float g, float u, float alpha, float limit) {
  if constexpr (ACT == 0) {
    const float gc = __builtin_amdgcn_fmed3f(g, 0.f, limit);
    const float uc = __builtin_amdgcn_fmed3f(u, -limit, limit);
    return gc * sigmoidf_(alpha * gc) * uc;
  } else {
    return g * sigmoidf_(g) * u;
  }
}

// 8 e2m1 codes (one 32-bit word, element 0 in the low nibble) times the block
// scale 2^(s - 127) -> 8 bf16 (element 0 in the low half of the first word).
// gfx950's v_cvt_scalef32_pk_bf16_fp4 converts the two codes of one byte
// (low nibble to the low half) with an fp32 scale; every product is a bf16
// number, so the result is exact.  The NaN scale (s = 255) is set explicitly.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32x4_t decode_e2m1x8(uint32_t codes, uint32_t s) {
  const float scale = __uint_as_float(s == 0 ? 0x00400000u : (s << 23));
  u32x4_t r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 0));
  r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 1));
  r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 2));
  r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 3));
  if (s == 255u) r = u32x4_t{0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u};
  return r;
}

// NJ = 32-column result tiles per wavefront (block columns BN = 64 NJ);
// BK = K elements per stage; NS / NSB = LDS stages of A / B.
template <int WF, bool GATED, int NJ, int BK, int NS, int NSB>
__global__ __launch_bounds__(kThreads, 1) void mfma_gemm_kernel(MfmaArgs a) {
  constexpr int BN = 64 * NJ;
  constexpr int CPR = BK / 8;             // 16-byte chunks per LDS row
  constexpr int SEG_ROWS = 1024 / (2 * BK);  // rows per 1 KB copy segment
  constexpr int RA = BM * CPR / kThreads; // copy instructions per wavefront and tile, A
  constexpr int RB = WF == WF_MXFP4 ? 0 : BN * CPR / kThreads;  // same, B (MXFP4: none)
  // MXFP4: code copies per wavefront and 4-tile group (8 rows x 128 B each)
  constexpr int RC = WF == WF_MXFP4 ? BN * 8 / kThreads : 0;
  static_assert(!GATED || NJ % 2 == 0, "gate|up pairs need an even number of column tiles");
  static_assert(NS >= 2 && NSB >= NS && NSB <= NS + 1, "LDS stages");
  static_assert(WF != WF_MXFP4 || NSB == NS, "MXFP4 weights use symmetric stages");
  static_assert(BM * CPR % kThreads == 0 && BN * CPR % kThreads == 0, "copy rounds");
  static_assert(NS <= 5 && NSB <= 5, "stage variables");
  // One LDS variable per stage: the compiler tells copies into one stage from
  // reads of another only by the variable they address (see the pipeline).
  // Unused stages (size 8) are never referenced and take no LDS.
  __shared__ uint16_t lds_a0[BM * BK], lds_a1[BM * BK], lds_a2[NS > 2 ? BM * BK : 8],
      lds_a3[NS > 3 ? BM * BK : 8], lds_a4[NS > 4 ? BM * BK : 8];
  __shared__ uint16_t lds_b0[BN * BK], lds_b1[BN * BK], lds_b2[NSB > 2 ? BN * BK : 8],
      lds_b3[NSB > 3 ? BN * BK : 8], lds_b4[NSB > 4 ? BN * BK : 8];
  // MXFP4 (every wait drains the copies anyway): one array per operand
  __shared__ uint16_t lds_mx_a[NS][BM * BK], lds_mx_b[NS][BN * BK];
  __shared__ uint16_t lds_mx_code[WF == WF_MXFP4 ? BN * 64 : 8];  // codes of 4 tiles, 128 B per row
  auto stage_a = [&](int st) __attribute__((always_inline)) -> uint16_t* {
    if constexpr (WF == WF_MXFP4) return lds_mx_a[st];
    if constexpr (NS > 4) {
      if (st == 4) return lds_a4;
    }
    if constexpr (NS > 3) {
      if (st == 3) return lds_a3;
    }
    if constexpr (NS > 2) {
      if (st == 2) return lds_a2;
    }
    return st == 0 ? lds_a0 : lds_a1;
  };
  auto stage_b = [&](int st) __attribute__((always_inline)) -> uint16_t* {
    if constexpr (WF == WF_MXFP4) return lds_mx_b[st];
    if constexpr (NSB > 4) {
      if (st == 4) return lds_b4;
    }
    if constexpr (NSB > 3) {
      if (st == 3) return lds_b3;
    }
    if constexpr (NSB > 2) {
      if (st == 2) return lds_b2;
    }
    return st == 0 ? lds_b0 : lds_b1;
  };

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
  int a_row[RA];
#pragma unroll
  for (int i = 0; i < RA; ++i) {
    const int r = SEG_ROWS * (4 * i + wv) + ld_sub;
    const int gr = r0 + r < r_end ? r0 + r : r0;
    a_row[i] = a.row_token ? a.row_token[gr] : gr;
  }
  constexpr int NBR = RB > RC ? RB : RC;  // B row rounds (bf16 copies or MXFP4 code copies)
  constexpr int RBX = NBR > 0 ? NBR : 1;
  int b_row[RBX];
#pragma unroll
  for (int i = 0; i < NBR; ++i) {
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

  // MXFP4: the codes of 4 K tiles (128 bytes of each B row) are copied into
  // lds_mx_code (8 rows x 128 B per instruction, like the bf16 weights; the
  // 16-byte chunks of row r are XOR-swizzled by r & 7); thread t < BN then
  // decodes row t of each tile from there with the tile's two scale bytes,
  // which it loads a tile ahead.
  bool mx_row_ok = false;
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
    mx_row_ok = tid < BN && wrow < N;
    const size_t row = (size_t)e * a.N + (wrow < N ? wrow : n0);
    mx_scales = (up ? a.s1 : a.s0) + row * (K / 32);
  }
  static_assert(WF != WF_MXFP4 || BK == 64, "MXFP4 stages hold 64 elements");
  uint32_t mxsc = 0x7f7fu;  // scale bytes of the next tile to decode (low: first 32 elements)

  // Every copy of a tile issues exactly RA (A) and RB (B) instructions per
  // wavefront (the K tail copies clamped, valid addresses and is zeroed after
  // it lands), so the counted waits below are exact.
  // logical chunk that lane slot ld_phys of round i holds (inverse of swz)
  auto ld_chunk_of = [&](int i) __attribute__((always_inline)) {
    const int row = SEG_ROWS * (4 * i + wv) + ld_sub;
    return (swz<BK>(row, ld_phys) - row * BK) >> 3;  // XOR is an involution
  };
  // round i of the copies of A / (dense) B tile kt into the stage at As / Bs.
  // (The stage pointer comes from the caller: a lambda that calls stage_a()
  // from inside another lambda makes this hipcc's host pass drop the kernel
  // stubs without a diagnostic.)
  auto copy_a = [&](int kt, uint16_t* As, int i) __attribute__((always_inline)) {
    const int k = min(kt * BK + 8 * ld_chunk_of(i), K - 8);
    __builtin_amdgcn_global_load_lds(a.a + (size_t)a_row[i] * a.lda + k, As + (4 * i + wv) * 512, 16, 0, 0);
  };
  auto copy_b = [&](int kt, uint16_t* Bs, int i) __attribute__((always_inline)) {
    const int k = min(kt * BK + 8 * ld_chunk_of(i), K - 8);
    const uint16_t* wsrc = (b_row[i] & 1) ? w_up : w_gate;
    __builtin_amdgcn_global_load_lds(wsrc + (size_t)(b_row[i] >> 1) * K + k, Bs + (4 * i + wv) * 512, 16, 0, 0);
  };
  auto issue_a = [&](int kt, int sa) __attribute__((always_inline)) {
    uint16_t* As = stage_a(sa);
#pragma unroll
    for (int i = 0; i < RA; ++i) copy_a(kt, As, i);
  };
  // MXFP4: copy the codes of 4-tile group g into lds_mx_code.  Chunks past
  // the row end copy the row's first chunk instead (decoded as zeros).
  auto mx_copy_codes = [&](int g, uint16_t* Cs) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < RC; ++i) {
      const int logical = ld_phys ^ (ld_sub & 7);  // the row's r & 7 is ld_sub
      int off = 128 * g + 16 * logical;
      if (off + 16 > K / 2) off = 0;
      const uint8_t* src = ((b_row[i] & 1) ? a.c1 : a.c0) + ((size_t)e * a.N + (b_row[i] >> 1)) * (K / 2) + off;
      __builtin_amdgcn_global_load_lds(src, Cs + (4 * i + wv) * 512, 16, 0, 0);
    }
  };
  auto issue_b = [&](int kt, int sb) __attribute__((always_inline)) {
    if constexpr (WF == WF_MXFP4) {
      // the tile's two scale bytes: one 2-byte load when K % 64 == 0 (rows of
      // K / 32 bytes keep it aligned), else byte loads of the halves inside K
      const int k0 = kt * BK;
      if ((K & 63) == 0 && k0 + 64 <= K) {
        mxsc = *reinterpret_cast<const uint16_t*>(mx_scales + k0 / 32);
      } else {
        const uint32_t b0 = k0 < K ? (uint32_t)mx_scales[k0 / 32] : 127u;
        const uint32_t b1 = k0 + 32 < K ? (uint32_t)mx_scales[k0 / 32 + 1] : 127u;
        mxsc = b0 | (b1 << 8);
      }
      if (kt % 4 == 0) mx_copy_codes(kt / 4, lds_mx_code);
    } else {
      uint16_t* Bs = stage_b(sb);
#pragma unroll
      for (int i = 0; i < RB; ++i) copy_b(kt, Bs, i);
    }
  };
  // MXFP4 only: decode tile t (row tid) from lds_mx_code into stage sb.  The
  // first tile of a group waits for the group's copies and meets the other
  // wavefronts first (the copies land in LDS asynchronously).
  auto finish_b = [&](int t, int sb) __attribute__((always_inline)) {
    if constexpr (WF == WF_MXFP4) {
      if (t % 4 == 0) {
        wait_vmcnt<0>();
        barrier_lds();
      }
      uint16_t* Bs = stage_b(sb);
      if (tid < BN) {
        const int q = t & 3, sw = tid & 7;
        const u32x4_t c0 = *reinterpret_cast<const u32x4_t*>(lds_mx_code + tid * 64 + ((2 * q) ^ sw) * 8);
        const u32x4_t c1 = *reinterpret_cast<const u32x4_t*>(lds_mx_code + tid * 64 + ((2 * q + 1) ^ sw) * 8);
        const bool ok0 = mx_row_ok && t * BK < K, ok1 = mx_row_ok && t * BK + 32 < K;
        const u32x4_t z = {0u, 0u, 0u, 0u};
        const uint32_t s0 = mxsc & 0xffu, s1 = (mxsc >> 8) & 0xffu;
        *reinterpret_cast<u32x4_t*>(Bs + swz<BK>(tid, 0)) = ok0 ? decode_e2m1x8(c0.x, s0) : z;
        *reinterpret_cast<u32x4_t*>(Bs + swz<BK>(tid, 1)) = ok0 ? decode_e2m1x8(c0.y, s0) : z;
        *reinterpret_cast<u32x4_t*>(Bs + swz<BK>(tid, 2)) = ok0 ? decode_e2m1x8(c0.z, s0) : z;
        *reinterpret_cast<u32x4_t*>(Bs + swz<BK>(tid, 3)) = ok0 ? decode_e2m1x8(c0.w, s0) : z;
        *reinterpret_cast<u32x4_t*>(Bs + swz<BK>(tid, 4)) = ok1 ? decode_e2m1x8(c1.x, s1) : z;
        *reinterpret_cast<u32x4_t*>(Bs + swz<BK>(tid, 5)) = ok1 ? decode_e2m1x8(c1.y, s1) : z;
        *reinterpret_cast<u32x4_t*>(Bs + swz<BK>(tid, 6)) = ok1 ? decode_e2m1x8(c1.z, s1) : z;
        *reinterpret_cast<u32x4_t*>(Bs + swz<BK>(tid, 7)) = ok1 ? decode_e2m1x8(c1.w, s1) : z;
      }
    }
  };
  // zero the chunks of the tile past K (the last tile only)
  auto zero_tail = [&](int kt, int sa, int sb) __attribute__((always_inline)) {
    uint16_t* As = stage_a(sa);
    uint16_t* Bs = stage_b(sb);
#pragma unroll
    for (int i = 0; i < RA; ++i)
      if (kt * BK + 8 * ld_chunk_of(i) >= K)
        *reinterpret_cast<u32x4_t*>(As + (4 * i + wv) * 512 + 8 * lane) = u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < RB; ++i)
      if (kt * BK + 8 * ld_chunk_of(i) >= K)
        *reinterpret_cast<u32x4_t*>(Bs + (4 * i + wv) * 512 + 8 * lane) = u32x4_t{0u, 0u, 0u, 0u};
  };

  f32x16_t acc[4][NJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  // ---- pipeline.  Copies are issued in batches, one per tile boundary: the
  // batch of slot s holds A(s + NS) then B(s + NSB) (each if it exists), and
  // slot s's batch is issued in the last 16-wide K step of tile s, right after
  // the barrier that ends all reads of tile s (its last fragments are already
  // in registers) -- into the stages tile s used.  The prologue issues the
  // batches of slots -NSB .. -1.  Before the barrier of tile kt the block
  // needs tile kt+1, whose last instruction is A(kt+1) (B(kt+1) when NSB ==
  // NS); only the instructions issued after it may still be in flight.  In
  // steady state those are B(kt+1+NSB-NS) (NSB > NS) and NS - 2 whole
  // batches; near the end of K the block simply waits for everything.
  // Within a tile the fragments of step kk+1 are read while step kk
  // multiplies (two register sets).  sched_barrier(0) keeps the compiler from
  // sinking those reads below the MFMAs they are meant to overlap.
  //
  // The compiler adds its own wait before an LDS read for every copy in
  // flight into the LDS variable that read addresses.  Each stage is its own
  // variable, and the steady loop is unrolled by P = lcm(NS, NSB) tiles so
  // that every stage index is a compile-time constant: the reads of tile kt+1
  // then never wait for the copies into other stages (with run-time indices
  // they would wait for all copies).
  constexpr int KK = BK / 16;
  static_assert(KK % 2 == 0, "fragment double buffering needs an even step count");
  constexpr int kSteadyWait = (NSB > NS ? RB : 0) + (NS - 2) * (RA + RB);
  constexpr int kPrologueWait = (NSB > NS ? RB : 0) + (NS - 1) * (RA + RB);
  constexpr int P = NS == NSB ? NS : NS * NSB;  // NSB = NS + 1 is coprime to NS
  const int ktiles = (K + BK - 1) / BK;
  const int tail_tile = (K % BK) != 0 ? ktiles - 1 : -1;
  const int fr = lane & 31, fk = lane >> 5;

  bf16x8_t fa[2][4], fb[2][NJ];
  // fragment r of step kk (r < 4: A row block r; else B column block r - 4)
  auto load_frag = [&](const uint16_t* As, const uint16_t* Bs, int kk, int buf, int r) __attribute__((always_inline)) {
    if (r < 4)
      fa[buf][r] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(As + swz<BK>(wm * 128 + 32 * r + fr, 2 * kk + fk)));
    else
      fb[buf][r - 4] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(Bs + swz<BK>(wn * 32 * NJ + 32 * (r - 4) + fr, 2 * kk + fk)));
  };
  auto load_frags = [&](int sa, int sb, int kk, int buf) __attribute__((always_inline)) {
    const uint16_t* As = stage_a(sa);
    const uint16_t* Bs = stage_b(sb);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      fa[buf][i] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(As + swz<BK>(wm * 128 + 32 * i + fr, 2 * kk + fk)));
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      fb[buf][j] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(Bs + swz<BK>(wn * 32 * NJ + 32 * j + fr, 2 * kk + fk)));
  };

#pragma unroll
  for (int s = -NSB; s < 0; ++s) {
    if (s + NS >= 0 && s + NS < ktiles) issue_a(s + NS, s + NS);
    if (s + NSB < ktiles) {
      issue_b(s + NSB, s + NSB);
      // MXFP4: tile 0 is decoded now; every later tile t at the end of tile
      // t-1, a whole tile after its codes were requested
      if (s + NSB == 0) finish_b(0, 0);
    }
  }
  if (WF != WF_MXFP4 && ktiles >= NSB) wait_vmcnt<(WF == WF_MXFP4 ? 0 : kPrologueWait)>();
  else wait_vmcnt<0>();
  barrier_lds();
  if (tail_tile == 0) {
    zero_tail(0, 0, 0);
    barrier_lds();
  }
  load_frags(0, 0, 0, 0);
  // One K tile.  STEADY: every batch up to slot kt is whole and tile kt+1 is
  // no tail, so the step runs without branches and with a counted wait.
  // PH >= 0: kt % P == PH (stage indices are constants); PH < 0: run time.
  auto tile_step = [&](int kt, auto steady_tag, auto phase_tag) __attribute__((always_inline)) {
    constexpr bool STEADY = decltype(steady_tag)::value;
    constexpr int PH = decltype(phase_tag)::value;
    const int sa = PH >= 0 ? PH % NS : kt % NS;            // stages of tile kt (and of the batch issued now)
    const int sb = PH >= 0 ? PH % NSB : kt % NSB;
    const int sa1 = PH >= 0 ? (PH + 1) % NS : (kt + 1) % NS;  // stages of tile kt+1
    const int sb1 = PH >= 0 ? (PH + 1) % NSB : (kt + 1) % NSB;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const int cur = kk & 1;
      if (kk + 1 < KK) {
        // this step's fragments were read a whole MFMA run ago; waiting for
        // them here keeps the wait from also covering the reads issued next
        wait_lgkmcnt0();
        if constexpr (kInterleaveLds != 0) {
          const uint16_t* As = stage_a(sa);
          const uint16_t* Bs = stage_b(sb);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
              acc[i][j] = mfma_32x32x16(fa[cur][i], fb[cur][j], acc[i][j]);
              const int m = i * NJ + j;
              if (kInterleaveLds == 1 && m < 4 + NJ) load_frag(As, Bs, kk + 1, cur ^ 1, m);
              if (kInterleaveLds == 2 && (m & 1) && (m >> 1) < 4 + NJ) load_frag(As, Bs, kk + 1, cur ^ 1, m >> 1);
              __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
          for (int r = kInterleaveLds == 1 ? 4 * NJ : 2 * NJ; r < 4 + NJ; ++r) load_frag(As, Bs, kk + 1, cur ^ 1, r);
          continue;
        }
        load_frags(sa, sb, kk + 1, cur ^ 1);
      } else if (STEADY || kt + 1 < ktiles) {
        // MXFP4: decode tile kt+1 into its stage (free since the barrier that
        // ended tile kt-1) from the codes requested at that barrier
        if constexpr (WF == WF_MXFP4) finish_b(kt + 1, sb1);
        if (STEADY && WF != WF_MXFP4) wait_vmcnt<(WF == WF_MXFP4 ? 0 : kSteadyWait)>();
        else wait_vmcnt<0>();
        barrier_lds();  // tile kt+1 is in LDS; every wavefront is done reading tile kt
        if (!STEADY && kt + 1 == tail_tile) {
          zero_tail(kt + 1, sa1, sb1);
          barrier_lds();
        }
        if (STEADY && kInterleave && WF != WF_MXFP4) {
          // the batch alternates with this step's MFMAs
          uint16_t* As = stage_a(sa);
          uint16_t* Bs = stage_b(sb);
          const uint16_t* As1 = stage_a(sa1);
          const uint16_t* Bs1 = stage_b(sb1);
          if constexpr (!kBoundaryReadsInterleaved) load_frags(sa1, sb1, 0, cur ^ 1);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
              acc[i][j] = mfma_32x32x16(fa[cur][i], fb[cur][j], acc[i][j]);
              const int m = i * NJ + j;
              if (m < RA) copy_a(kt + NS, As, m);
              else if (m - RA < RB) copy_b(kt + NSB, Bs, m - RA);
              if (kBoundaryReadsInterleaved && m < 4 + NJ) load_frag(As1, Bs1, 0, cur ^ 1, m);
              __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
          for (int m = 4 * NJ; m < RA + RB; ++m) {
            if (m < RA) copy_a(kt + NS, As, m);
            else copy_b(kt + NSB, Bs, m - RA);
          }
          if constexpr (kBoundaryReadsInterleaved) {
#pragma unroll
            for (int r = 4 * NJ; r < 4 + NJ; ++r) load_frag(As1, Bs1, 0, cur ^ 1, r);
          }
          continue;
        }
        if (STEADY || kt + NS < ktiles) issue_a(kt + NS, sa);
        if (STEADY || kt + NSB < ktiles) issue_b(kt + NSB, sb);
        load_frags(sa1, sb1, 0, cur ^ 1);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = mfma_32x32x16(fa[cur][i], fb[cur][j], acc[i][j]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // P consecutive steady tiles starting at kt0 (kt0 % P == 0)
  auto steady_group = [&](int kt0, auto self, auto phase_tag) __attribute__((always_inline)) {
    constexpr int PH = decltype(phase_tag)::value;
    if constexpr (PH < P) {
      tile_step(kt0 + PH, std::true_type{}, phase_tag);
      self(kt0, self, std::integral_constant<int, PH + 1>{});
    }
  };
  int kt = 0;
  const int steady_end = ktiles - NSB - (tail_tile >= 0 ? 1 : 0);
  if constexpr (WF == WF_MXFP4) {
    // MXFP4 waits for every copy at each tile boundary anyway (its weight
    // codes come through registers), and unrolling would spill registers
    for (; kt < steady_end; ++kt) tile_step(kt, std::true_type{}, std::integral_constant<int, -1>{});
  } else {
    for (; kt + P <= steady_end; kt += P) steady_group(kt, steady_group, std::integral_constant<int, 0>{});
  }
  for (; kt < ktiles; ++kt) tile_step(kt, std::false_type{}, std::integral_constant<int, -1>{});
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
  // this lane's first output row, and whether the whole tile is inside the
  // expert's rows and the N columns (then the stores need no bounds check)
  const int lane_row = r0 + wm * 128 + 4 * fk + c4;
  uint16_t* const lane_out = a.out + (size_t)lane_row * a.ldo + (fr & ~3);
  const bool tile_inside = r0 + BM <= r_end && n0 + (GATED ? BN / 2 : BN) <= N;
  float bv0[OJ], bv1[OJ];
  int colj[OJ];
#pragma unroll
  for (int j = 0; j < OJ; ++j) {
    colj[j] = GATED ? n0 + 32 * (2 * wn + j) : n0 + wn * 32 * NJ + 32 * j;
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
  if (L.wfmt == WF_MXFP4) mfma_gemm_kernel<WF_MXFP4, true, 4, kBKMx, kStagesMx, kStagesMx><<<grid, kThreads, 0, s>>>(m);
  else mfma_gemm_kernel<WF_BF16, true, 4, kBK, kStages, kStagesB><<<grid, kThreads, 0, s>>>(m);
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
  // Column tile width 192 or 256, whichever copies fewer bytes into LDS:
  // per K step a row tile copies (256 + width) rows for each column tile.
  // (The copies bound this kernel, so padded columns cost less than narrow
  // tiles: d = 2880 takes 12 tiles of 256 rather than 15 of 192.)
  const int t192 = (L.d + 191) / 192, t256 = (L.d + 255) / 256;
  const bool narrow = t192 * (256 + 192) < t256 * (256 + 256);
  m.n_tiles = narrow ? t192 : t256;
  const dim3 grid(grid_for(max_row_tiles(L) * m.n_tiles));
  if (L.wfmt == WF_MXFP4) {
    if (narrow) mfma_gemm_kernel<WF_MXFP4, false, 3, kBKMx, kStagesMx, kStagesMx><<<grid, kThreads, 0, s>>>(m);
    else mfma_gemm_kernel<WF_MXFP4, false, 4, kBKMx, kStagesMx, kStagesMx><<<grid, kThreads, 0, s>>>(m);
  } else {
    if (narrow) mfma_gemm_kernel<WF_BF16, false, 3, kBK, kStages, kStagesB><<<grid, kThreads, 0, s>>>(m);
    else mfma_gemm_kernel<WF_BF16, false, 4, kBK, kStages, kStagesB><<<grid, kThreads, 0, s>>>(m);
  }
  return hipGetLastError();
}

}  // namespace moe
