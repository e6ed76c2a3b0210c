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
// MI355X the copies are bound by the L2 requests a CU keeps in flight more
// than by how far ahead they are issued: NSB = NS = 2 by default, NSB = 3 for
// launches whose experts average two or more row tiles (1% faster there).
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
// x).
#include <type_traits>

#include "gemm_common.h"
#include "permute_common.h"
#include "route_mfma.h"

namespace moe {
namespace {

using namespace gemm;

// Tuning knobs (compile-time; -D overrides for sweeps).
#ifndef MOE_GEMM_GROUP_M
#define MOE_GEMM_GROUP_M 8
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
#ifndef MOE_GEMM_WAVES_N
#define MOE_GEMM_WAVES_N 2
#endif
// Wavefronts along N: 2 (4 wavefronts of 128 x 128, one per SIMD) or 4 (8
// wavefronts of 128 x 64, two per SIMD).
constexpr int kWavesN = MOE_GEMM_WAVES_N;
// A rows past a tile's last row copy a row of zeros (1) or the tile's first
// row (0).
#ifndef MOE_GEMM_ZERO_ROWS
#define MOE_GEMM_ZERO_ROWS 1
#endif
constexpr bool kZeroRows = MOE_GEMM_ZERO_ROWS != 0;




// NJ = 32-column result tiles per wavefront; WN = wavefronts along N (2 x WN
// wavefronts, block columns BN = 32 NJ WN); BK = K elements per stage;
// NS / NSB = LDS stages of A / B.
// One block tile: rows [r0, r_end) of expert e (the shared expert is e = E),
// column tile n_tile.
template <bool GATED, int NJ, int BK, int NS, int NSB, int WN>
__device__ __forceinline__ void mfma_gemm_tile(const MfmaArgs& a, int e, int r0, int r_end, int n_tile) {
  constexpr int NW = 2 * WN;              // wavefronts
  constexpr int NT = 64 * NW;             // threads
  constexpr int BN = 32 * NJ * WN;
  constexpr int CPR = BK / 8;             // 16-byte chunks per LDS row
  constexpr int SEG_ROWS = 1024 / (2 * BK);  // rows per 1 KB copy segment
  constexpr int RA = BM * CPR / NT;       // copy instructions per wavefront and tile, A
  constexpr int RB = BN * CPR / NT;       // same, B
  static_assert(!GATED || NJ % 2 == 0, "gate|up pairs need an even number of column tiles");
  static_assert(NS >= 2 && NSB >= NS && NSB <= NS + 1, "LDS stages");
  static_assert(BM * CPR % NT == 0 && BN * CPR % NT == 0, "copy rounds");
  static_assert(NS <= 5 && NSB <= 5, "stage variables");
  // One LDS variable per stage: the compiler tells copies into one stage from
  // reads of another only by the variable they address (see the pipeline).
  // Unused stages (size 8) are never referenced and take no LDS.
  __shared__ uint16_t lds_a0[BM * BK], lds_a1[BM * BK], lds_a2[NS > 2 ? BM * BK : 8],
      lds_a3[NS > 3 ? BM * BK : 8], lds_a4[NS > 4 ? BM * BK : 8];
  __shared__ uint16_t lds_b0[BN * BK], lds_b1[BN * BK], lds_b2[NSB > 2 ? BN * BK : 8],
      lds_b3[NSB > 3 ? BN * BK : 8], lds_b4[NSB > 4 ? BN * BK : 8];
  auto stage_a = [&](int st) __attribute__((always_inline)) -> uint16_t* {
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

  const bool shared = e >= a.E;
  const int N = shared ? a.N_sh : a.N;
  const int K = shared ? a.K_sh : a.K;
  const int n0 = n_tile * (GATED ? BN / 2 : BN);
  if (n0 >= N) return;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv / WN, wn = wv % WN;

  // ---- copy coordinates.  In round i, wavefront wv fills the 1 KB LDS
  // segment NW i + wv: lane l writes 16-byte slot l, i.e. row
  // SEG_ROWS (NW i + wv) + l / CPR, stored chunk l % CPR, which holds the
  // logical chunk that swz() maps there.  Rows past the expert's last row (A)
  // copy the zero row a.zrow (a_row -1), else the tile's first row; rows past
  // N (B) copy a valid row.  They only feed outputs that the epilogue drops
  // (zeros keep the matrix cores' operands quiet: measured 0.5% faster on the
  // 8192-token layer).
  const int ld_sub = lane / CPR;
  const int ld_phys = lane % CPR;
  int a_row[RA];
#pragma unroll
  for (int i = 0; i < RA; ++i) {
    const int r = SEG_ROWS * (NW * i + wv) + ld_sub;
    const bool dead = r0 + r >= r_end;
    const int gr = dead ? r0 : r0 + r;
    a_row[i] = dead && a.zrow ? -1 : a.row_token ? a.row_token[gr] : gr - a.a_row0;
  }
  int b_row[RB];
#pragma unroll
  for (int i = 0; i < RB; ++i) {
    const int r = SEG_ROWS * (NW * i + wv) + ld_sub;
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

  // Every copy of a tile issues exactly RA (A) and RB (B) instructions per
  // wavefront (the K tail copies clamped, valid addresses and is zeroed after
  // it lands), so the counted waits below are exact.
  // logical chunk that lane slot ld_phys of round i holds (inverse of swz)
  auto ld_chunk_of = [&](int i) __attribute__((always_inline)) {
    const int row = SEG_ROWS * (NW * i + wv) + ld_sub;
    return (swz<BK>(row, ld_phys) - row * BK) >> 3;  // XOR is an involution
  };
  // round i of the copies of A / (dense) B tile kt into the stage at As / Bs.
  // (The stage pointer comes from the caller: a lambda that calls stage_a()
  // from inside another lambda makes this hipcc's host pass drop the kernel
  // stubs without a diagnostic.)
  auto copy_a = [&](int kt, uint16_t* As, int i) __attribute__((always_inline)) {
    const int k = min(kt * BK + 8 * ld_chunk_of(i), K - 8);
    const uint16_t* row = a_row[i] >= 0 ? a.a + (size_t)a_row[i] * a.lda : a.zrow;
    __builtin_amdgcn_global_load_lds(row + k, As + (NW * i + wv) * 512, 16, 0, 0);
  };
  auto copy_b = [&](int kt, uint16_t* Bs, int i) __attribute__((always_inline)) {
    const int k = min(kt * BK + 8 * ld_chunk_of(i), K - 8);
    const uint16_t* wsrc = (b_row[i] & 1) ? w_up : w_gate;
    __builtin_amdgcn_global_load_lds(wsrc + (size_t)(b_row[i] >> 1) * K + k, Bs + (NW * i + wv) * 512, 16, 0, 0);
  };
  auto issue_a = [&](int kt, int sa) __attribute__((always_inline)) {
    uint16_t* As = stage_a(sa);
#pragma unroll
    for (int i = 0; i < RA; ++i) copy_a(kt, As, i);
  };
  auto issue_b = [&](int kt, int sb) __attribute__((always_inline)) {
    uint16_t* Bs = stage_b(sb);
#pragma unroll
    for (int i = 0; i < RB; ++i) copy_b(kt, Bs, i);
  };
  // zero the chunks of the tile past K (the last tile only)
  auto zero_tail = [&](int kt, int sa, int sb) __attribute__((always_inline)) {
    uint16_t* As = stage_a(sa);
    uint16_t* Bs = stage_b(sb);
#pragma unroll
    for (int i = 0; i < RA; ++i)
      if (kt * BK + 8 * ld_chunk_of(i) >= K)
        *reinterpret_cast<u32x4_t*>(As + (NW * i + wv) * 512 + 8 * lane) = u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < RB; ++i)
      if (kt * BK + 8 * ld_chunk_of(i) >= K)
        *reinterpret_cast<u32x4_t*>(Bs + (NW * i + wv) * 512 + 8 * lane) = u32x4_t{0u, 0u, 0u, 0u};
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
    if (s + NSB < ktiles) issue_b(s + NSB, s + NSB);
  }
  if (ktiles >= NSB) wait_vmcnt<kPrologueWait>();
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
        if (STEADY) wait_vmcnt<kSteadyWait>();
        else wait_vmcnt<0>();
        barrier_lds();  // tile kt+1 is in LDS; every wavefront is done reading tile kt
        if (!STEADY && kt + 1 == tail_tile) {
          zero_tail(kt + 1, sa1, sb1);
          barrier_lds();
        }
        if (STEADY && kInterleave) {
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
  for (; kt + P <= steady_end; kt += P) steady_group(kt, steady_group, std::integral_constant<int, 0>{});
  for (; kt < ktiles; ++kt) tile_step(kt, std::false_type{}, std::integral_constant<int, -1>{});
  wait_vmcnt<0>();
  barrier_lds();  // every wavefront is done with the stages before they are reused

  // ---- epilogue: bias (+ activation) in registers, bf16 stores
  store_tile<GATED, NJ, WN>(a, acc, e, shared, N, n0, r0, r_end, wm, wn, lane);
}

// The tiles of experts [e_first, e_end) in the XCD-aware order, one per block.
template <bool GATED, int NJ, int BK, int NS, int NSB, int WN>
__global__ __launch_bounds__(128 * WN, 1) void mfma_gemm_kernel(MfmaArgs a) {
  int m_tile, n_tile;
  if (!block_tile<kGroupM>(a, m_tile, n_tile)) return;
  const int4 desc = reinterpret_cast<const int4*>(a.tile_desc)[m_tile];
  mfma_gemm_tile<GATED, NJ, BK, NS, NSB, WN>(a, desc.x, desc.y, desc.z, n_tile);
}

// ---- the shared expert beside the router and the permutation ---------------
// The shared expert's T rows (sorted rows [P, P + T), P = T k, one per token
// in token order) need neither the routing nor the permutation.  Its gate|up
// tiles therefore run in the router's launch and its down tiles in the
// permutation's, on CUs those leave idle, and the routed launches are whole
// waves of routed tiles.  The first blocks of such a launch are router (or
// permutation) blocks; block n_other + i is shared tile i: row tile i % mt,
// column tile i / mt (mt row tiles: with n_other a multiple of 8, the tiles
// of one row tile stay on one XCD and share its A panel through that L2).
template <bool GATED, int NJ>
__device__ __forceinline__ void shared_tile(const MfmaArgs& a, int i, int P, int T) {
  const int mt = (T + BM - 1) / BM;
  const int m = i % mt, n = i / mt;
  if (n >= a.n_tiles) return;
  mfma_gemm_tile<GATED, NJ, kBK, 2, 2, 2>(a, a.E, P + BM * m, P + T, n);
}

// router blocks (4 wavefronts each, tree sum) and the shared expert's gate|up
template <int EG>
__global__ __launch_bounds__(256, 1) void route_shared_gate_up_kernel(RouteArgs ra, int n_route, MfmaArgs a, int P, int T) {
  if ((int)blockIdx.x < n_route) {
    route_mfma_block<EG, 4, true, false>(ra, blockIdx.x);
    return;
  }
  shared_tile<true, 4>(a, blockIdx.x - n_route, P, T);
}

// permutation blocks and the shared expert's down product
template <int NJ>
__global__ __launch_bounds__(256, 1) void permute_shared_down_kernel(PermuteArgs pa, int n_perm, MfmaArgs a, int P, int T) {
  if ((int)blockIdx.x < n_perm) {
    permute_block(pa, blockIdx.x);
    return;
  }
  shared_tile<false, NJ>(a, blockIdx.x - n_perm, P, T);
}

}  // namespace

namespace {
MfmaArgs gate_up_args(const Layer& L, const Work& W, int e_first, int e_end) {
  MfmaArgs m = base_args(L, W);
  m.e_first = e_first;
  m.e_end = e_end;
  m.a = static_cast<const uint16_t*>(L.x);
  m.lda = L.d;
  m.row_token = W.row_token;
  m.w0 = static_cast<const uint16_t*>(L.wg);
  m.w1 = static_cast<const uint16_t*>(L.wu);
  m.bias0 = static_cast<const uint16_t*>(L.bg);
  m.bias1 = static_cast<const uint16_t*>(L.bu);
  m.sh_w0 = static_cast<const uint16_t*>(L.sh_wg);
  m.sh_w1 = static_cast<const uint16_t*>(L.sh_wu);
  m.N = L.F; m.K = L.d; m.N_sh = L.F_sh; m.K_sh = L.d;
  m.out = static_cast<uint16_t*>(W.h);
  m.ldo = L.F_max();
  m.n_tiles = (L.F_max() + 127) / 128;
  m.zrow = kZeroRows ? static_cast<const uint16_t*>(W.zrow) : nullptr;
  return m;
}

// Column tile width 192 or 256, whichever copies fewer bytes into LDS:
// per K step a row tile copies (256 + width) rows for each column tile.
// (The copies bound this kernel, so padded columns cost less than narrow
// tiles: d = 2880 takes 12 tiles of 256 rather than 15 of 192.)
bool down_narrow(const Layer& L) {
  const int t192 = (L.d + 191) / 192, t256 = (L.d + 255) / 256;
  return t192 * (256 + 192) < t256 * (256 + 256);
}

MfmaArgs down_args(const Layer& L, const Work& W, int e_first, int e_end) {
  MfmaArgs m = base_args(L, W);
  m.e_first = e_first;
  m.e_end = e_end;
  m.a = static_cast<const uint16_t*>(W.h);
  m.lda = L.F_max();
  m.row_token = nullptr;
  m.w0 = static_cast<const uint16_t*>(L.wd);
  m.bias0 = static_cast<const uint16_t*>(L.bd);
  m.sh_w0 = static_cast<const uint16_t*>(L.sh_wd);
  m.N = L.d; m.K = L.F; m.N_sh = L.d; m.K_sh = L.F_sh;
  m.out = static_cast<uint16_t*>(W.y);
  m.ldo = L.d;
  m.n_tiles = down_narrow(L) ? (L.d + 191) / 192 : (L.d + 255) / 256;
  m.zrow = kZeroRows ? static_cast<const uint16_t*>(W.zrow) : nullptr;
  return m;
}

// Weight copies a tile further ahead (a third LDS stage for B, all 160 KB of
// LDS) where the routed experts average at least two 256-row tiles, so
// that an expert's weight panels serve several row tiles: on the 8192-token
// layer (32 experts, 1024 rows each on average) gate|up 1119-1126 against
// 1134-1139 us; on GLM-sized layers (192 rows per expert, one row tile each)
// it measured slower (0.476-0.487 against 0.473-0.477 ms per step).
bool deep_weight_stages(const Layer& L, int e_first, int e_end) {
  return kStagesB == 2 && e_first < L.E && e_end >= L.E && (long long)L.T * L.k >= 2LL * BM * L.E;
}

hipError_t gate_up_mfma(const Layer& L, const Work& W, hipStream_t s, int e_first, int e_end) {
  const MfmaArgs m = gate_up_args(L, W, e_first, e_end);
  const dim3 grid(grid_for(max_row_tiles(L, e_first, e_end) * m.n_tiles));
  if (kWavesN == 4) mfma_gemm_kernel<true, 2, kBK, kStages, kStagesB, 4><<<grid, 512, 0, s>>>(m);
  else if (deep_weight_stages(L, e_first, e_end)) mfma_gemm_kernel<true, 4, kBK, kStages, 3, 2><<<grid, 256, 0, s>>>(m);
  else mfma_gemm_kernel<true, 4, kBK, kStages, kStagesB, 2><<<grid, 256, 0, s>>>(m);
  return hipGetLastError();
}

hipError_t down_mfma(const Layer& L, const Work& W, hipStream_t s, int e_first, int e_end) {
  const MfmaArgs m = down_args(L, W, e_first, e_end);
  const dim3 grid(grid_for(max_row_tiles(L, e_first, e_end) * m.n_tiles));
  if (down_narrow(L)) mfma_gemm_kernel<false, 3, kBK, kStages, kStagesB, 2><<<grid, 256, 0, s>>>(m);
  else if (kWavesN == 4) mfma_gemm_kernel<false, 2, kBK, kStages, kStagesB, 4><<<grid, 512, 0, s>>>(m);
  else if (deep_weight_stages(L, e_first, e_end)) mfma_gemm_kernel<false, 4, kBK, kStages, 3, 2><<<grid, 256, 0, s>>>(m);
  else mfma_gemm_kernel<false, 4, kBK, kStages, kStagesB, 2><<<grid, 256, 0, s>>>(m);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_gate_up_mfma(const Layer& L, const Work& W, hipStream_t s, bool routed_only) {
  return gate_up_mfma(L, W, s, 0, routed_only ? L.E : L.n_experts_all());
}
hipError_t launch_down_mfma(const Layer& L, const Work& W, hipStream_t s, bool routed_only) {
  return down_mfma(L, W, s, 0, routed_only ? L.E : L.n_experts_all());
}
hipError_t launch_gate_up_mfma_shared(const Layer& L, const Work& W, hipStream_t s) {
  return gate_up_mfma(L, W, s, L.E, L.E + 1);
}
hipError_t launch_down_mfma_shared(const Layer& L, const Work& W, hipStream_t s) {
  return down_mfma(L, W, s, L.E, L.E + 1);
}

hipError_t launch_route_shared_gate_up(const Layer& L, const Work& W, hipStream_t s) {
  const RouteArgs ra = route_args(L, W);
  const int n_route = (L.T + kMfmaTokens - 1) / kMfmaTokens;
  MfmaArgs m = gate_up_args(L, W, L.E, L.E + 1);
  const int P = L.T * L.k;
  m.row_token = nullptr;  // shared row P + t is token t
  m.a_row0 = P;
  m.zrow = nullptr;  // the permutation writes the zero row later
  const dim3 grid(n_route + (L.T + BM - 1) / BM * m.n_tiles);
  if (L.E <= 16) route_shared_gate_up_kernel<1><<<grid, 256, 0, s>>>(ra, n_route, m, P, L.T);
  else if (L.E <= 32) route_shared_gate_up_kernel<2><<<grid, 256, 0, s>>>(ra, n_route, m, P, L.T);
  else if (L.E <= 64) route_shared_gate_up_kernel<4><<<grid, 256, 0, s>>>(ra, n_route, m, P, L.T);
  else route_shared_gate_up_kernel<8><<<grid, 256, 0, s>>>(ra, n_route, m, P, L.T);  // E <= kSharedBesideMaxE
  return hipGetLastError();
}

hipError_t launch_permute_shared_down(const Layer& L, const Work& W, hipStream_t s) {
  const PermuteArgs pa = permute_args(L, W);
  const int n_perm = (L.T + kPermuteTokens - 1) / kPermuteTokens;
  MfmaArgs m = down_args(L, W, L.E, L.E + 1);
  m.zrow = nullptr;  // written by this launch's permutation blocks
  const int P = L.T * L.k;
  const dim3 grid(n_perm + (L.T + BM - 1) / BM * m.n_tiles);
  if (down_narrow(L)) permute_shared_down_kernel<3><<<grid, 256, 0, s>>>(pa, n_perm, m, P, L.T);
  else permute_shared_down_kernel<4><<<grid, 256, 0, s>>>(pa, n_perm, m, P, L.T);
  return hipGetLastError();
}

}  // namespace moe
