// Grouped expert GEMMs on the gfx950 scaled MFMA (v_mfma_scale_f32_32x32x64_f8f6f4):
// MXFP8 activations (E4M3 codes and e8m0 scales from mx_quant_kernel) times
// MXFP4 (e2m1) or MXFP8 (E4M3) expert weights with e8m0 scales (OCP
// Microscaling Formats v1.0), fp32 accumulation.  The block scales are
// applied by the matrix core.
//
//   gate|up:  h[r][f] = act(xq[t] . Wg[e][f] + bg[e][f], xq[t] . Wu[e][f] + bu[e][f])  (t = row_token[r])
//   down:     y[r][n] = hq[r] . Wd[e][n] + bd[e][n]
//
// (MaxText GPT-OSS weight mapping "MOE EXPERTS"; glm4_moe_lite.go
// SwitchMLP.Forward; the GGUF page's MXFP4 expert weights; MXFP8 as in
// glm4_moe_lite.go quantizationParams.)
//
// Block tile 256 rows x 256 columns, 4 wavefronts of 128 x 128 (4 x 4 results
// of 32 x 32), the tile order, bias and activation epilogue of the bf16 GEMM.
// K goes in stages of 128 through two LDS buffers per operand, filled by
// global -> LDS copies a stage ahead: A 256 rows x 128 code bytes (rows
// swizzled as the bf16 kernel's 64-wide bf16 stages), B 256 rows x 64 (e2m1,
// as its 32-wide stages) or 128 (E4M3) code bytes, and each row's 4 scale
// bytes of the stage.
// A stage is two MFMA steps of 64 k.  The activation rows are the quantizer's
// output: lda (a multiple of 128) bytes a row, zero codes past K, so whole
// stages are always in bounds; weight copies past a row's end are clamped.
#include <type_traits>

#include "gemm_common.h"

namespace moe {
namespace {

using namespace gemm;

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));

constexpr int kGroupM = 4;               // row tiles walked together within an XCD
// A rows past a tile's last row copy the workspace's zero row (1) or the
// tile's first row (0).
#ifndef MOE_MX_ZERO_ROWS
#define MOE_MX_ZERO_ROWS 1
#endif
constexpr bool kMxZeroRows = MOE_MX_ZERO_ROWS != 0;
constexpr int NJ = 4;                    // 32-column results per wavefront
constexpr int BN = 64 * NJ;              // 256 block columns
constexpr int BKX = 128;                 // K elements per stage
constexpr int RA = BM * 8 / kThreads;    // 16-byte A copies per thread and stage (8)
constexpr int RSB = BN * 2 / kThreads;   // B scale dwords (2)
// weight code bytes of a B row per stage (WB = weight bits: 4 e2m1, 8 E4M3),
// 16-byte B copies per thread and stage, and copy instructions per stage
template <int WB> constexpr int b_row_bytes() { return WB * BKX / 8; }
template <int WB> constexpr int b_copies() { return BN * (b_row_bytes<WB>() / 16) / kThreads; }
template <int WB> constexpr int n_copies() { return RA + b_copies<WB>() + 1 + RSB; }
constexpr int kMaxRB = 8;  // array bound for the B copies (b_copies<8>())

// D (32 x 32) += A (32 x 64) * B (64 x 32) with block scales.  Lane
// l = 32 h + r supplies A row r: code bytes 0..15 hold k = 16 h .. +15 and
// bytes 16..31 hold k = 32 + 16 h .. +15; B column r: for E4M3 the same
// layout, for e2m1 16 bytes holding k = 32 h .. +31 (element 2i in the low
// nibble); byte SEL of sa / sb: the scale of A row r / B column r for
// k = 32 h .. +31.  The other scale bytes are ignored.  Result layout as
// mfma_32x32x16.
template <int SEL>
__device__ __forceinline__ f32x16_t mfma_mx(i32x8_t a, i32x4_t b, f32x16_t c, uint32_t sa, uint32_t sb) {
  const i32x8_t b8 = __builtin_shufflevector(b, b, 0, 1, 2, 3, -1, -1, -1, -1);  // e2m1 reads 4 registers
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b8, c, 0 /* A: E4M3 */, 4 /* B: E2M1 */, SEL, (int)sa,
                                                         SEL, (int)sb);
}
template <int SEL>
__device__ __forceinline__ f32x16_t mfma_mx(i32x8_t a, i32x8_t b, f32x16_t c, uint32_t sa, uint32_t sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0 /* A: E4M3 */, 0 /* B: E4M3 */, SEL, (int)sa,
                                                         SEL, (int)sb);
}

template <bool GATED, int WB>
__global__ __launch_bounds__(kThreads, 1) void mx_gemm_kernel(MfmaArgs a) {
  constexpr int BRB = b_row_bytes<WB>();      // B code bytes of a row per stage
  constexpr int RB = b_copies<WB>();          // 16-byte B copies per thread and stage
  constexpr int kCopies = n_copies<WB>();     // copy instructions per thread and stage
  constexpr int BCPR = BRB / 16;              // 16-byte chunks of a B row
  using bfrag_t = std::conditional_t<WB == 8, i32x8_t, i32x4_t>;
  // One LDS variable per stage (the compiler tells copies into one stage
  // from reads of another only by the variable they address).
  __shared__ uint16_t lds_a0[BM * 64], lds_a1[BM * 64];  // 128-byte rows
  __shared__ uint16_t lds_b0[BN * BRB / 2], lds_b1[BN * BRB / 2];  // BRB-byte rows
  __shared__ uint32_t lds_sa0[BM], lds_sa1[BM];          // A row r: scale bytes of the stage's 4 blocks
  __shared__ uint32_t lds_sb0[2 * BN], lds_sb1[2 * BN];  // B row r: the two aligned dwords holding them

  int m_tile, n_tile;
  if (!block_tile<kGroupM>(a, m_tile, n_tile)) return;
  const int4 desc = reinterpret_cast<const int4*>(a.tile_desc)[m_tile];
  const int e = desc.x;
  const int N = a.N, K = a.K;
  const int n0 = n_tile * (GATED ? BN / 2 : BN);
  if (n0 >= N) return;
  const int r0 = desc.y, r_end = desc.z;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv >> 1, wn = wv & 1;
  const int fr = lane & 31, fh = lane >> 5;
  const uint8_t* const aq = reinterpret_cast<const uint8_t*>(a.a);
  const uint32_t lda = (uint32_t)a.lda;

  // weight row of B tile row r (gate|up: 128 gate and the same 128 up rows
  // interleaved by 32), and whether it is an up row; rows past N read row n0
  auto b_row = [&](int r, bool& up) __attribute__((always_inline)) {
    int wrow;
    if constexpr (GATED) {
      wrow = n0 + 32 * (r >> 6) + (r & 31);
      up = (r & 63) >= 32;
    } else {
      wrow = n0 + r;
      up = false;
    }
    return wrow < N ? wrow : n0;
  };
  auto a_token = [&](int r) __attribute__((always_inline)) {
    const int gr = r0 + r < r_end ? r0 + r : r0;
    return a.row_token ? a.row_token[gr] : gr;
  };

  // ---- copy coordinates.  A round i: wavefront wv fills the 1 KB LDS
  // segment 4 i + wv, 8 rows of 128 bytes; lane l writes slot l % 8 of row
  // 8 (4 i + wv) + l / 8, which holds the logical chunk swz() maps there.
  // B round i: 1024 / BRB rows of BRB bytes, slot l % BCPR of row
  // (1024 / BRB) (4 i + wv) + l / BCPR.
  // Rows past the tile's last row copy the zero row (zoff: its byte offset
  // from the codes, both in the workspace), else the tile's first row.
  const uint32_t zoff = a.zrow ? (uint32_t)(reinterpret_cast<const uint8_t*>(a.zrow) - aq) : 0u;
  uint32_t a_off[RA];  // byte offset of the copied chunk in stage 0
#pragma unroll
  for (int i = 0; i < RA; ++i) {
    const int row = 8 * (4 * i + wv) + (lane >> 3);
    const int chunk = (swz<64>(row, lane & 7) - row * 64) >> 3;
    a_off[i] = (r0 + row >= r_end && a.zrow ? zoff : (uint32_t)a_token(row) * lda) + 16u * (uint32_t)chunk;
  }
  const uint32_t sa_off = (uint32_t)a_token(tid) * (lda / 32);  // A scales: thread tid copies row tid
  const int kb = K * WB / 8;  // code bytes of a weight row
  const size_t e_rows = (size_t)e * N;
  const uint8_t* const code_g = a.c0 + e_rows * kb;
  const uint8_t* const code_u = GATED ? a.c1 + e_rows * kb : code_g;
  // Copy round i reads the up tensor when its B tile rows r have
  // r % 64 >= 32, which for these row numbers is i odd (E4M3: 8 rows a
  // segment) or wv >= 2 (e2m1: 16 rows a segment), so the base is uniform
  // (written out in copy_m: a lambda called from inside another lambda makes
  // hipcc's host pass drop the kernel stubs).
  // (sized by a namespace constant: a local array whose bound is a local
  // constexpr of the template, captured by a lambda, also makes the host
  // pass drop the kernel stubs)
  static_assert(RB <= kMaxRB, "B copy rounds");
  uint32_t b_off[kMaxRB];  // byte offset of the row from its tensor's expert base
  uint32_t b_k[kMaxRB];    // byte offset of the copied chunk within the row's stage
#pragma unroll
  for (int i = 0; i < RB; ++i) {
    const int row = (1024 / BRB) * (4 * i + wv) + lane / BCPR;
    bool up;
    const int wrow = b_row(row, up);
    b_off[i] = (uint32_t)wrow * (uint32_t)kb;
    b_k[i] = 16u * (uint32_t)((swz<BRB / 2>(row, lane % BCPR) - row * (BRB / 2)) >> 3);
  }
  // B scales: dword q = 256 i + tid of a stage's table is dword q % 2 of the
  // aligned pair that holds B row q / 2's four scale bytes (its scale tensor
  // is 4-byte aligned, so the pair never starts before it); dwords past the
  // tensor's end are clamped to its last one (their bytes serve no block).
  const int ks = K / 32;
  const uintptr_t sc_g = reinterpret_cast<uintptr_t>(a.s0) + e_rows * ks;
  const uintptr_t sc_u = GATED ? reinterpret_cast<uintptr_t>(a.s1) + e_rows * ks : sc_g;
  const uintptr_t end_g = reinterpret_cast<uintptr_t>(a.s0) + (size_t)a.E * N * ks - 4;
  const uintptr_t end_u = GATED ? reinterpret_cast<uintptr_t>(a.s1) + (size_t)a.E * N * ks - 4 : end_g;
  uintptr_t sb_addr[RSB], sb_end[RSB];
#pragma unroll
  for (int i = 0; i < RSB; ++i) {
    const int q = 256 * i + tid;
    bool up;
    const int wrow = b_row(q >> 1, up);
    sb_addr[i] = (((up ? sc_u : sc_g) + (size_t)wrow * ks) & ~(uintptr_t)3) + 4 * (q & 1);
    sb_end[i] = up ? end_u : end_g;
  }
  // this lane's shift of each B fragment row's dword pair: byte 0 then holds
  // block fh of the stage and byte 2 block 2 + fh
  int sb_shift[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    bool up;
    const int wrow = b_row(wn * 128 + 32 * j + fr, up);
    sb_shift[j] = 8 * (int)(((up ? sc_u : sc_g) + (size_t)wrow * ks) & 3) + 8 * fh;
  }

  auto copy_m = [&](int kt, uint16_t* As, uint16_t* Bs, uint32_t* SAs, uint32_t* SBs, int m)
      __attribute__((always_inline)) {
    if (m < RA) {
      __builtin_amdgcn_global_load_lds(aq + (a_off[m] + (uint32_t)kt * BKX), As + (4 * m + wv) * 512, 16, 0, 0);
    } else if (m < RA + RB) {
      const int i = m - RA;
      const uint32_t k = min((uint32_t)kt * BRB + b_k[i], (uint32_t)kb - 16u);
      const bool up = GATED && (WB == 8 ? (i & 1) != 0 : wv >= 2);
      __builtin_amdgcn_global_load_lds((up ? code_u : code_g) + (b_off[i] + k), Bs + (4 * i + wv) * 512, 16, 0, 0);
    } else if (m == RA + RB) {
      __builtin_amdgcn_global_load_lds(a.as + (sa_off + 4u * (uint32_t)kt), SAs + 64 * wv, 4, 0, 0);
    } else {
      const int i = m - RA - RB - 1;
      const uintptr_t p0 = sb_addr[i] + 4 * (uintptr_t)kt;
      const uintptr_t p = p0 < sb_end[i] ? p0 : sb_end[i];
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(p), SBs + 256 * i + 64 * wv, 4, 0, 0);
    }
  };

  f32x16_t acc[4][NJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  // A fragments are single-buffered: row block i of the next step is read
  // right after the current step's last MFMA on it (the other row blocks'
  // MFMAs cover the read).  B fragments alternate between two sets by step.
  // E4M3 weights: B fragments single-buffered too (column block j refilled
  // right after the step's last MFMA on it), for registers
  constexpr int NBS = WB == 8 ? 1 : 2;
  i32x8_t fa[4];
  bfrag_t fb[NBS][NJ];
  uint32_t sa[4], sb[NJ], sb_n[NJ];
  // A fragment of row block i for step t
  auto read_a = [&](const uint16_t* As, int t, int i) __attribute__((always_inline)) {
    const int row = wm * 128 + 32 * i + fr;
    const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(As + swz<64>(row, 4 * t + fh));
    const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(As + swz<64>(row, 4 * t + 2 + fh));
    fa[i] = i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  };
  // B fragment of column block j for step t into set t (E4M3: the one set)
  auto read_b = [&](const uint16_t* Bs, int t, int j) __attribute__((always_inline)) {
    const int row = wn * 128 + 32 * j + fr;
    if constexpr (WB == 8) {
      const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(Bs + swz<64>(row, 4 * t + fh));
      const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(Bs + swz<64>(row, 4 * t + 2 + fh));
      fb[0][j] = i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    } else {
      fb[t][j] = __builtin_bit_cast(i32x4_t, *reinterpret_cast<const u32x4_t*>(Bs + swz<32>(row, 2 * t + fh)));
    }
  };
  // scale dword of A row block i / B column block j of a stage
  auto read_sa = [&](const uint32_t* SAs, int i) __attribute__((always_inline)) {
    return SAs[wm * 128 + 32 * i + fr] >> (8 * fh);
  };
  auto read_sb = [&](const uint32_t* SBs, int j) __attribute__((always_inline)) {
    const uint64_t v = *reinterpret_cast<const uint64_t*>(SBs + 2 * (wn * 128 + 32 * j + fr));
    return (uint32_t)(v >> sb_shift[j]);
  };
  auto mma = [&](int t, int i, int j) __attribute__((always_inline)) {
    if (t == 0) acc[i][j] = mfma_mx<0>(fa[i], fb[0][j], acc[i][j], sa[i], sb[j]);
    else acc[i][j] = mfma_mx<2>(fa[i], fb[NBS - 1][j], acc[i][j], sa[i], sb[j]);
  };

  const int ktiles = (K + BKX - 1) / BKX;
  const bool half_last = (K % BKX) != 0;  // K % 64 == 0: the last stage then has one step
  // prologue: stages 0 and 1
#pragma unroll
  for (int m = 0; m < kCopies; ++m) copy_m(0, lds_a0, lds_b0, lds_sa0, lds_sb0, m);
  if (ktiles > 1) {
#pragma unroll
    for (int m = 0; m < kCopies; ++m) copy_m(1, lds_a1, lds_b1, lds_sa1, lds_sb1, m);
    wait_vmcnt<kCopies>();
  } else {
    wait_vmcnt<0>();
  }
  barrier_lds();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    sa[i] = read_sa(lds_sa0, i);
    read_a(lds_a0, 0, i);
  }
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    sb[j] = read_sb(lds_sb0, j);
    read_b(lds_b0, 0, j);
  }

  // One stage.  STEADY: the stage after next exists, so its copies are
  // issued here and nothing branches; ST = kt % 2 is then a compile-time
  // constant (STc >= 0).  The tail stages take one code path with run-time
  // conditions around the barrier and the copies only: code paths that merge
  // with the accumulators live make the register allocator move them.
  // Step 1 of a last stage holding only 64 k still runs: its A codes are zero
  // (the quantizer pads each row), its A scales are byte 0 (2^-127), and its
  // B scale bytes, which lie past the row, are replaced by 127 (1.0), so it
  // adds exact zeros.
  auto stage_step = [&](int kt, auto st_tag, auto steady_tag) __attribute__((always_inline)) {
    constexpr int STc = decltype(st_tag)::value;
    constexpr bool STEADY = decltype(steady_tag)::value;
    const int ST = STc >= 0 ? STc : (kt & 1);
    uint16_t* const As = ST ? lds_a1 : lds_a0;
    uint16_t* const Bs = ST ? lds_b1 : lds_b0;
    uint32_t* const SAs = ST ? lds_sa1 : lds_sa0;
    uint32_t* const SBs = ST ? lds_sb1 : lds_sb0;
    const uint16_t* const As1 = ST ? lds_a0 : lds_a1;  // the next stage's buffers
    const uint16_t* const Bs1 = ST ? lds_b0 : lds_b1;
    const uint32_t* const SAs1 = ST ? lds_sa0 : lds_sa1;
    const uint32_t* const SBs1 = ST ? lds_sb0 : lds_sb1;
    // step 0; the step-1 fragments of this stage are read in between
    wait_lgkmcnt0();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        mma(0, i, j);
        if (i == (NBS == 2 ? 0 : 3)) read_b(Bs, 1, j);
        if (j == NJ - 1) read_a(As, 1, i);
        __builtin_amdgcn_sched_barrier(0);
      }
    wait_lgkmcnt0();
    const bool has_next = STEADY || kt + 1 < ktiles;
    const bool more = STEADY || kt + 2 < ktiles;
    if (has_next) {
      wait_vmcnt<0>();
      barrier_lds();  // stage kt+1 is in LDS; every wavefront is done reading stage kt
    } else if (half_last) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) sb[j] = (sb[j] & 0xff00ffffu) | (127u << 16);
    }
    // step 1, alternating with the copies of stage kt+2 into this stage's
    // buffers and the reads of stage kt+1's scales and step-0 fragments (in
    // the last stage these read a buffer that nothing writes any more)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        mma(1, i, j);
        const int m = i * NJ + j;
        if (m < kCopies && more) copy_m(kt + 2, As, Bs, SAs, SBs, m);
        // more copies than MFMAs (E4M3 weights): the last ones double up
        if (kCopies > 16 && m >= 32 - kCopies && more) copy_m(kt + 2, As, Bs, SAs, SBs, m + kCopies - 16);
        if (i == 0) sb_n[j] = read_sb(SBs1, j);
        if (i == (NBS == 2 ? 0 : 3)) read_b(Bs1, 0, j);
        if (j == NJ - 1) {
          read_a(As1, 0, i);
          sa[i] = read_sa(SAs1, i);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
    for (int j = 0; j < NJ; ++j) sb[j] = sb_n[j];
  };
  int kt = 0;
  for (; kt + 3 < ktiles; kt += 2) {
    stage_step(kt, std::integral_constant<int, 0>{}, std::true_type{});
    stage_step(kt + 1, std::integral_constant<int, 1>{}, std::true_type{});
  }
  for (; kt < ktiles; ++kt) stage_step(kt, std::integral_constant<int, -1>{}, std::false_type{});
  wait_vmcnt<0>();
  barrier_lds();

  // ---- epilogue: bias (+ activation) in registers, bf16 stores
  store_tile<GATED, NJ>(a, acc, e, false, N, n0, r0, r_end, wm, wn, lane);
}

// The zero row, if its byte offset from the codes fits the kernel's 32-bit
// row offsets (the codes' own offsets are checked below 2^32 by the library).
const uint16_t* zero_row_for(const Work& W, const uint8_t* codes) {
  if (!kMxZeroRows || !W.zrow) return nullptr;
  const uintptr_t z = reinterpret_cast<uintptr_t>(W.zrow), c = reinterpret_cast<uintptr_t>(codes);
  return z > c && z - c < (1ull << 32) - (1u << 16) ? static_cast<const uint16_t*>(W.zrow) : nullptr;
}

}  // namespace

hipError_t launch_gate_up_mx(const Layer& L, const Work& W, hipStream_t s) {
  MfmaArgs m = base_args(L, W);
  m.a = reinterpret_cast<const uint16_t*>(W.xq);
  m.as = W.xs;
  m.zrow = zero_row_for(W, W.xq);
  m.lda = mx_row_bytes(L.d);
  m.row_token = W.row_token;
  m.c0 = L.wg_codes; m.s0 = L.wg_scales;
  m.c1 = L.wu_codes; m.s1 = L.wu_scales;
  m.bias0 = static_cast<const uint16_t*>(L.bg);
  m.bias1 = static_cast<const uint16_t*>(L.bu);
  m.N = L.F; m.K = L.d;
  m.out = static_cast<uint16_t*>(W.h);
  m.ldo = L.F_max();
  m.n_tiles = (L.F + BN / 2 - 1) / (BN / 2);
  const dim3 grid(grid_for(max_row_tiles(L) * m.n_tiles));
  if (L.wfmt == WF_MXFP8) mx_gemm_kernel<true, 8><<<grid, kThreads, 0, s>>>(m);
  else mx_gemm_kernel<true, 4><<<grid, kThreads, 0, s>>>(m);
  return hipGetLastError();
}

hipError_t launch_down_mx(const Layer& L, const Work& W, hipStream_t s) {
  MfmaArgs m = base_args(L, W);
  m.a = reinterpret_cast<const uint16_t*>(W.hq);
  m.as = W.hs;
  m.zrow = zero_row_for(W, W.hq);
  m.lda = mx_row_bytes(L.F);
  m.row_token = nullptr;
  m.c0 = L.wd_codes; m.s0 = L.wd_scales;
  m.bias0 = static_cast<const uint16_t*>(L.bd);
  m.N = L.d; m.K = L.F;
  m.out = static_cast<uint16_t*>(W.y);
  m.ldo = L.d;
  m.n_tiles = (L.d + BN - 1) / BN;
  const dim3 grid(grid_for(max_row_tiles(L) * m.n_tiles));
  if (L.wfmt == WF_MXFP8) mx_gemm_kernel<false, 8><<<grid, kThreads, 0, s>>>(m);
  else mx_gemm_kernel<false, 4><<<grid, kThreads, 0, s>>>(m);
  return hipGetLastError();
}

}  // namespace moe
