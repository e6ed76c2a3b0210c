// Grouped expert GEMMs with low-bit expert weights on bf16 MFMA.
//
//   gate|up:  h[r][f] = act(x[t] . Wg[e][f] + bg[e][f], x[t] . Wu[e][f] + bu[e][f])
//   down:     y[r][n] = h[r] . Wd[e][n] + bd[e][n]
//   MXFP4:    W[e][n][k] = e2m1(code[e][n][k]) * 2^(scale[e][n][k / 32] - 127)
//   NVFP4:    W[e][n][k] = e2m1(code[e][n][k]) * e4m3(scale[e][n][k / 16]) * tensor_scale
//   affine:   W[e][n][k] = scale[e][n][k / G] * q[e][n][k] + bias[e][n][k / G]
//             (4-bit codes with G = 32, 8-bit codes with G = 64)
//
// (MaxText GPT-OSS weight mapping "MOE EXPERTS"; the weight format of the
// MXFP4 GPT-OSS checkpoints; OCP Microscaling Formats v1.0 for e2m1 / e8m0;
// glm4_moe_lite.go SwitchMLP / quantizationParams for the affine experts and
// the NVFP4 group of 16.)
//
// MXFP4 products e2m1 * 2^s are bf16 numbers, so those operands are exact;
// affine weights are computed in fp32 (one fma) and rounded once to bf16.
//
// Same tile geometry, tile order and epilogue as the dense bf16 kernel, but
// the weights stay 4-bit until they reach registers: the codes are copied
// into LDS (a quarter of the bf16 bytes), each wavefront reads its own code
// fragments from there and converts them into the bf16 B operands of the
// MFMAs, in the shadow of the previous step's MFMAs: gfx950's
// v_cvt_scalef32_pk_bf16_fp4 for MXFP4 (its scale is a power of two); for
// NVFP4 v_cvt_scalef32_pk_f32_fp4 with scale 1, a multiply by the block's
// fp32 scale (its E4M3 scale times the tensor scale; a lane's 32 codes of a
// tile span two blocks of 16, steps 0-1 and 2-3) and a bf16 pack;
// byte-to-float conversions, one fma
// with the group's scale and bias, and a bf16 pack for affine codes.
//
// K permutation.  v_mfma_f32_32x32x16_bf16 takes 8 k values from each lane
// half h = lane / 32.  Within a 64-wide K tile, half h of step s (0..3) holds
// k = 32 h + 8 s .. +7 for both operands (the MFMA sums over k in any order as
// long as A and B agree): a lane's B codes for the whole tile are then one
// 16-byte (4-bit) or 32-byte (8-bit) piece of its weight row under one scale
// (and bias), and its A fragment of step s is 16-byte chunk 4 h + s of its
// LDS row.
//
// 128 bytes of each weight row's codes (4 K tiles of 4-bit, 2 of 8-bit codes)
// are copied as one group,
// 8 rows x 128 B per 1 KB instruction, into one of two group buffers; the
// copies of group g + 1 are issued when tile 4 g starts, into the buffer that
// group g - 1 used.  FAST kernels (K % 64 == 0, scale tensors 4-byte aligned
// in base and size) copy the scales of each row and group like the codes (as
// the aligned dwords that hold them; affine: scales and biases) and run every
// K tile but the last with the same branch-free step.  The general kernel
// loads each lane's scales into registers a tile ahead and handles a K tail.
#include <type_traits>

#include "gemm_common.h"

#ifndef MOE_MX_GROUP_M
#define MOE_MX_GROUP_M 4
#endif

namespace moe {
namespace {

using namespace gemm;

constexpr int kGroupM = MOE_MX_GROUP_M;  // row tiles walked together within an XCD
// Wavefronts along N for MXFP4 weights: 4 (8 wavefronts of 128 x 64, two per
// SIMD, so one wavefront's waits on LDS and conversions overlap the other's
// MFMAs) or 2 (4 of 128 x 128).  The other formats keep 2: their decode needs
// more registers, and at two wavefronts per SIMD they spill (INT4 gate|up 240
// -> 347 us; MXFP4: 661 -> 656 us, down ~6% faster).
#ifndef MOE_LOWBIT_MX4_WAVES_N
#define MOE_LOWBIT_MX4_WAVES_N 4
#endif
constexpr int kMx4WavesN = MOE_LOWBIT_MX4_WAVES_N;
constexpr int BK = 64;                   // K elements per A stage and per decode tile
constexpr int kCodeRowBytes = 128;       // bytes of a weight row's codes per copy group
// weight formats
constexpr int kFmtMx4 = 0, kFmtAff4 = 1, kFmtAff8 = 2, kFmtNv4 = 3;
// kinds of K-tile step (see tile_step)
constexpr int kSteady = 0, kGeneral = 1, kLast = 2, kFinal = 3;
template <int V> using int_c = std::integral_constant<int, V>;
// Bound of the A row-offset array (its first RA entries are used): an array
// sized by a local constexpr that depends on a template parameter, captured
// by a lambda, makes this hipcc's host pass drop the kernel stubs.
constexpr int kMaxRA = 8;

// Stored position of 16-byte chunk c of code row r in LDS: XOR-swizzled by
// bits 1..3 of the row, so that the 16-byte reads of any 16 consecutive rows
// (same logical chunk; rows alternate between the two 128-byte halves of a
// 256-byte bank window) fall in 16 distinct 16-byte slots.
__device__ __forceinline__ int code_chunk(int row, int c) { return c ^ ((row >> 1) & 7); }

// e8m0 block scale as the fp32 factor of the conversion (s = 0: 2^-127, a
// denormal; s = 255, NaN, is handled by the caller).
__device__ __forceinline__ float scale_factor(uint32_t s) { return __uint_as_float(s == 0 ? 0x00400000u : (s << 23)); }

// Byte p of a word of e2m1 codes (low nibble first) times the scale -> two
// bf16 (low nibble in the low half).  p must fold to a constant.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cvt_fp4_pair(uint32_t codes, float scale, int p) {
  bf16x2_t r;
  if (p == 0) r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 0);
  else if (p == 1) r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 1);
  else if (p == 2) r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 2);
  else r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 3);
  return __builtin_bit_cast(uint32_t, r);
}

// bf16 pair (lo in the low half) of two fp32 values, one v_cvt_pk_bf16_f32
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}
// Byte p of a word of e2m1 codes (low nibble first) as two exact fp32
// values.  p must fold to a constant.  (The scaled conversions apply a
// power-of-two scale, as MX blocks have; NVFP4 scales are multiplied after.)
typedef float f32x2v_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ f32x2v_t fp4_pair_f32(uint32_t codes, int p) {
  if (p == 0) return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 0);
  if (p == 1) return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 1);
  if (p == 2) return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 2);
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 3);
}
// Value of an E4M3 code (sign, 4 exponent bits with bias 7, 3 mantissa bits;
// exponent 0 is subnormal, S.1111.111 is NaN), exact in fp32.
__device__ __forceinline__ float e4m3_value(uint32_t b) {
  const uint32_t ex = (b >> 3) & 15u, m = b & 7u;
  float v = ex == 0 ? (float)m * 0.001953125f : __uint_as_float(((ex + 120u) << 23) | (m << 20));
  v = (b & 0x7fu) == 0x7fu ? __uint_as_float(0x7fc00000u) : v;
  return (b & 0x80u) ? -v : v;
}
// byte b of w as a float (v_cvt_f32_ubyte<b>); b must fold to a constant
__device__ __forceinline__ float ubyte(uint32_t w, int b) { return static_cast<float>((w >> (8 * b)) & 0xffu); }

// WN = wavefronts along N (2 x WN wavefronts, each 128 rows x 32 NJ columns).
template <int FMT, bool GATED, int NJ, bool FAST, int WN>
__global__ __launch_bounds__(128 * WN, 1) void lowbit_gemm_kernel(MfmaArgs a) {
  constexpr int NW = 2 * WN;        // wavefronts
  constexpr int NTH = 64 * NW;      // threads
  constexpr bool MX = FMT == kFmtMx4;
  constexpr bool NV = FMT == kFmtNv4;
  constexpr bool FP4 = MX || NV;                   // e2m1 codes with byte scales
  constexpr int CB = FMT == kFmtAff8 ? 8 : 4;      // code bits
  constexpr int kTilesPerGroup = kCodeRowBytes / (BK * CB / 8);  // 4 (4-bit) or 2 (8-bit)
  constexpr int QG = MX ? 32 : NV ? 16 : (CB == 4 ? 32 : 64);  // elements per scale
  constexpr bool SCALE_LDS = FAST;                 // scales (and biases) copied into LDS per group
  constexpr int NT = FP4 ? 1 : 2;                  // scale tables: e8m0 / E4M3 scales; affine scales and biases
  constexpr int EB = FP4 ? 1 : 2;                  // bytes per table element (scale byte / bf16)
  constexpr int SBY = EB * BK * kTilesPerGroup / QG;  // bytes of one row and code group in one table
  constexpr int kScaleDw = (SBY + 3) / 4 + 1;      // aligned dwords that hold them (2-byte aligned start)
  constexpr int BN = 32 * NJ * WN;
  constexpr int CPR = BK / 8;               // 16-byte chunks per A row
  constexpr int SEG_ROWS = 1024 / (2 * BK); // A rows per 1 KB copy segment
  constexpr int RA = BM * CPR / NTH;        // A copy instructions per wavefront and tile
  constexpr int RC = BN * kCodeRowBytes / 1024 / NW;  // code copy instructions per wavefront and group
  static_assert(!GATED || NJ % 2 == 0, "gate|up pairs need an even number of column tiles");
  static_assert(BN * kCodeRowBytes % 4096 == 0, "code copy rounds");
  constexpr int KK = BK / 16;  // MFMA steps per tile
  static_assert(KK == 4, "a lane's 16-byte code piece covers the 4 steps of a tile");
  constexpr int NM = 4 * NJ;   // MFMAs per step
  constexpr int RS = (BN * kScaleDw + NTH - 1) / NTH;  // copy rounds per wavefront, group and table

  // A stages are separate variables (the compiler tells copies into one from
  // reads of the other only by the variable they address); the steady loop
  // is unrolled by 2 so that their indices are compile-time constants.
  __shared__ uint16_t lds_a0[BM * BK], lds_a1[BM * BK];
  __shared__ uint16_t lds_code[2][BN * kCodeRowBytes / 2];
  // scale tables of two code groups; table t, row r: bytes 4 kScaleDw r .. + 4 kScaleDw - 1
  __shared__ uint32_t lds_scale[2][NT][SCALE_LDS ? RS * NTH : 1];
  auto stage_a = [&](int st) __attribute__((always_inline)) -> uint16_t* { return st == 0 ? lds_a0 : lds_a1; };

  int m_tile, n_tile;
  if (!block_tile<kGroupM>(a, m_tile, n_tile)) return;
  const int4 desc = reinterpret_cast<const int4*>(a.tile_desc)[m_tile];
  const int e = desc.x;
  if (e >= a.E) return;  // the launch covers routed experts only; kept as a guard
  const int N = a.N;
  const int K = a.K;
  const int n0 = n_tile * (GATED ? BN / 2 : BN);
  if (n0 >= N) return;
  const int r0 = desc.y;
  const int r_end = desc.z;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv / WN, wn = wv % WN;
  const int fr = lane & 31, fk = lane >> 5;

  // B row r of the block is weight row n0 + 32 (r / 64) + r % 32 of the gate
  // (r % 64 < 32) or up tensor in the gate|up stage, n0 + r otherwise.  Rows
  // past N use row n0 (their outputs are dropped).
  auto clamp_row = [&](int wrow) __attribute__((always_inline)) { return wrow < N ? wrow : n0; };

  // ---- copy coordinates (as the dense kernel: in round i wavefront wv fills
  // the 1 KB LDS segment NW i + wv, lane l its 16-byte slot l).
  const int ld_sub = lane / CPR;
  const int ld_phys = lane % CPR;
  // element offset of each copied A row (the A operand is under 2^31
  // elements; the library checks)
  static_assert(RA <= kMaxRA, "A copy rounds");
  uint32_t a_row[kMaxRA];
#pragma unroll
  for (int i = 0; i < RA; ++i) {
    const int r = SEG_ROWS * (NW * i + wv) + ld_sub;
    const int gr = r0 + r < r_end ? r0 + r : r0;
    a_row[i] = (uint32_t)(a.row_token ? a.row_token[gr] : gr) * (uint32_t)a.lda;
  }
  // The expert's code and scale tensors (gate, up); byte offsets within one
  // expert fit 32 bits (the library rejects larger experts).
  const int code_bytes = K * CB / 8;  // of one weight row
  const uint8_t* const code_gate = a.c0 + (size_t)e * N * code_bytes;
  const uint8_t* const code_up = GATED ? a.c1 + (size_t)e * N * code_bytes : code_gate;
  // MXFP4 / NVFP4: scale bytes [E, N, K / QG]
  const uint8_t* const scale_gate = FP4 ? a.s0 + (size_t)e * N * (K / QG) : nullptr;
  const uint8_t* const scale_up = FP4 && GATED ? a.s1 + (size_t)e * N * (K / QG) : scale_gate;
  // affine: bf16 scales and biases [E, N, K / QG]
  const uint16_t* const qs_gate = FP4 ? nullptr : reinterpret_cast<const uint16_t*>(a.s0) + (size_t)e * N * (K / QG);
  const uint16_t* const qs_up = !FP4 && GATED ? reinterpret_cast<const uint16_t*>(a.s1) + (size_t)e * N * (K / QG) : qs_gate;
  const uint16_t* const qb_gate = FP4 ? nullptr : a.qb0 + (size_t)e * N * (K / QG);
  const uint16_t* const qb_up = !FP4 && GATED ? a.qb1 + (size_t)e * N * (K / QG) : qb_gate;
  // Code copy round i: lane l copies stored chunk l % 8 of B row
  // r = 8 NW i + code_r (code_r = 8 wv + l / 8 < 8 NW), i.e. weight row
  // n0 + 32 (r / 64) + r % 32 of the gate (r % 64 < 32) or up tensor in the
  // gate|up stage, n0 + r otherwise.  Bits 1..3 of the B row do not depend
  // on i, nor does the logical chunk the slot holds.
  const int code_r = 8 * wv + (lane >> 3);
  const uint32_t code_lane = 16u * (uint32_t)code_chunk(code_r, lane & 7);
  // this lane's fragment rows: B row wn 32 NJ + 32 j + fr of the block, i.e.
  // weight row n0 + 16 NJ wn + 32 (j / 2) + fr of the gate (j even) or up
  // tensor in the gate|up stage, n0 + 32 NJ wn + 32 j + fr otherwise
  auto frag_row = [&](int j) __attribute__((always_inline)) {
    return GATED ? n0 + 16 * NJ * wn + 32 * (j / 2) + fr : n0 + 32 * NJ * wn + 32 * j + fr;
  };
  const int code_off0 = (wn * 32 * NJ + fr) * (kCodeRowBytes / 2);  // uint16 offset of fragment row j = 0
  const int code_x = (wn * 32 * NJ + fr) >> 1 & 7;  // row hash of the fragment rows (32 j keeps it)

  const int ktiles = (K + BK - 1) / BK;
  const int tail_tile = (K % BK) != 0 ? ktiles - 1 : -1;

  auto copy_a = [&](int kt, uint16_t* As, int i) __attribute__((always_inline)) {
    const int row = SEG_ROWS * (NW * i + wv) + ld_sub;
    const int chunk = (swz<BK>(row, ld_phys) - row * BK) >> 3;  // logical chunk of this slot
    const int k = min(kt * BK + 8 * chunk, K - 8);
    __builtin_amdgcn_global_load_lds(a.a + (a_row[i] + (uint32_t)k), As + (NW * i + wv) * 512, 16, 0, 0);
  };
  auto issue_a = [&](int kt, int sa) __attribute__((always_inline)) {
    uint16_t* As = stage_a(sa);
#pragma unroll
    for (int i = 0; i < RA; ++i) copy_a(kt, As, i);
  };
  // codes of group g into buffer g % 2 (pieces past the row end copy the
  // row's first piece; the tiles that would use them mask them)
  auto issue_codes = [&](int g) __attribute__((always_inline)) {
    uint16_t* Cs = lds_code[g & 1];
    const uint32_t base = kCodeRowBytes * g;
    const uint32_t piece = base + code_lane + 16 <= (uint32_t)code_bytes ? base + code_lane : 0u;
#pragma unroll
    for (int i = 0; i < RC; ++i) {
      const int r = 8 * NW * i + code_r;
      const int wrow = clamp_row(GATED ? n0 + 32 * (r >> 6) + (r & 31) : n0 + r);
      const uint8_t* src = (GATED && (r & 63) >= 32) ? code_up : code_gate;
      __builtin_amdgcn_global_load_lds(src + ((uint32_t)wrow * (uint32_t)code_bytes + piece), Cs + (NW * i + wv) * 512, 16, 0, 0);
    }
  };
  // Tensor t of the scale tables (MXFP4: e8m0 scales; affine: scales, then
  // biases) of the gate (or down) and up weights, with the expert's offset.
  auto table = [&](int t, bool up) __attribute__((always_inline)) -> uintptr_t {
    const uint8_t* base = t == 0 ? (up ? a.s1 : a.s0) : reinterpret_cast<const uint8_t*>(up ? a.qb1 : a.qb0);
    return reinterpret_cast<uintptr_t>(base) + (size_t)e * N * (K / QG) * EB;
  };
  // FAST: the SBY bytes of code group g of every B row in each table, as the
  // kScaleDw aligned dwords that hold them, into scale buffer g % 2 (dword q
  // of a table is dword q % kScaleDw of row q / kScaleDw; rows past BN repeat
  // row BN - 1 into padding).  Dwords past the end of a tensor are clamped to
  // its last one (their bytes belong to no group of K).
  auto issue_scales = [&](int g) __attribute__((always_inline)) {
    const size_t tensor_bytes = (size_t)a.E * N * (K / QG) * EB;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      uint32_t* Ss = lds_scale[g & 1][t];
      const uintptr_t t_gate = table(t, false), t_up = GATED ? table(t, true) : t_gate;
      const uintptr_t end_gate = t_gate - (size_t)e * N * (K / QG) * EB + tensor_bytes - 4;
      const uintptr_t end_up = t_up - (size_t)e * N * (K / QG) * EB + tensor_bytes - 4;
#pragma unroll
      for (int i = 0; i < RS; ++i) {
        const int q = 64 * (NW * i + wv) + lane;
        const int r = min(q / kScaleDw, BN - 1);
        const bool up = GATED && (r & 63) >= 32;
        const int wrow = clamp_row(GATED ? n0 + 32 * (r >> 6) + (r & 31) : n0 + r);
        const uintptr_t row = (up ? t_up : t_gate) + (size_t)wrow * (K / QG) * EB + (size_t)SBY * g;
        const uintptr_t dw = min((row & ~(uintptr_t)3) + 4 * (q % kScaleDw), up ? end_up : end_gate);
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(dw), Ss + 64 * (NW * i + wv), 4, 0, 0);
      }
    }
  };
  // FAST: byte offset of this lane's fragment row j in scale table t (the
  // row's piece starts (row address & 3) bytes into its first dword)
  int sc_at[SCALE_LDS ? NT : 1][NJ];
  if constexpr (SCALE_LDS) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const uintptr_t row = table(t, GATED && (j & 1)) + (size_t)clamp_row(frag_row(j)) * (K / QG) * EB;
        sc_at[t][j] = kScaleDw * 4 * (wn * 32 * NJ + 32 * j + fr) + (int)(row & 3);
      }
  }
  // scales of tile kt for this lane's half: FAST from the scale buffer,
  // else from the tensors into registers a tile ahead (a half past K loads
  // the row's last scale; take_scales replaces it).  Affine: the bf16 scale
  // in the low and the bf16 bias in the high half of sraw; NVFP4: the scale
  // bytes of the half's two blocks of 16 in bytes 0 and 1.
  uint32_t sraw[NJ];
  auto load_scales = [&](int kt) __attribute__((always_inline)) {
    if constexpr (SCALE_LDS) {
      // element (BK (kt % TPG) + 32 fk) / QG of the row's group piece, behind
      // the piece's offset within its first aligned dword
      const int el = (BK * (kt % kTilesPerGroup) + 32 * fk) / QG;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        uint32_t v = 0;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const uint8_t* Sb = reinterpret_cast<const uint8_t*>(lds_scale[(kt / kTilesPerGroup) & 1][t]);
          const int at = sc_at[t][j] + EB * el;
          uint32_t x;
          if constexpr (NV) x = (uint32_t)Sb[at] | ((uint32_t)Sb[at + 1] << 8);
          else x = EB == 1 ? (uint32_t)Sb[at] : (uint32_t)*reinterpret_cast<const uint16_t*>(Sb + at);
          v |= x << (16 * t);
        }
        sraw[j] = v;
      }
    } else if constexpr (NV) {
      const int gi = min((BK * kt + 32 * fk) / 16, K / 16 - 2);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const uint8_t* p = ((GATED && (j & 1)) ? scale_up : scale_gate) + (uint32_t)clamp_row(frag_row(j)) * (uint32_t)(K / 16) + gi;
        sraw[j] = (uint32_t)p[0] | ((uint32_t)p[1] << 8);
      }
    } else if constexpr (!MX) {
      const int gi = min((BK * kt + 32 * fk) / QG, K / QG - 1);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const uint32_t at = (uint32_t)clamp_row(frag_row(j)) * (uint32_t)(K / QG) + gi;
        const bool up = GATED && (j & 1);
        sraw[j] = (uint32_t)(up ? qs_up : qs_gate)[at] | ((uint32_t)(up ? qb_up : qb_gate)[at] << 16);
      }
    } else {
      const int cb = min(2 * kt + fk, K / 32 - 1);
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        sraw[j] = ((GATED && (j & 1)) ? scale_up : scale_gate)[(uint32_t)clamp_row(frag_row(j)) * (uint32_t)(K / 32) + cb];
    }
  };
  float scf[NJ];      // scale factors of the current tile (NVFP4: of steps 0-1)
  float scf2[NV ? NJ : 1];  // NVFP4: scale factors of steps 2-3
  float sbi[FP4 ? 1 : NJ];  // affine: biases of the current tile
  uint32_t nan_j = 0; // MXFP4 / NVFP4, bit j: a NaN scale in the current tile
  // scales of tile kt from sraw (a half past K: scale 1 (MXFP4 byte 127),
  // affine scale and bias 0, with zero codes either way)
  auto take_scales = [&](int kt) __attribute__((always_inline)) {
    const bool past = !FAST && BK * kt + 32 * fk >= K;
    if constexpr (NV) {
      nan_j = 0;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const uint32_t sb = past ? 0x3838u : sraw[j];
        const float ts = (GATED && (j & 1)) ? a.ts1 : a.ts0;
        scf[j] = e4m3_value(sb & 0xffu) * ts;
        scf2[j] = e4m3_value(sb >> 8) * ts;
        nan_j |= ((sb & 0x7fu) == 0x7fu || (sb & 0x7f00u) == 0x7f00u ? 1u : 0u) << j;
      }
    } else if constexpr (MX) {
      nan_j = 0;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const uint32_t sb = past ? 127u : sraw[j];
        scf[j] = scale_factor(sb);
        nan_j |= (sb == 255u ? 1u : 0u) << j;
      }
    } else {
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        scf[j] = past ? 0.f : bf16_to_f32(static_cast<uint16_t>(sraw[j] & 0xffffu));
        sbi[j] = past ? 0.f : bf16_to_f32(static_cast<uint16_t>(sraw[j] >> 16));
      }
    }
  };
  // this lane's code pieces of tile kt (zero for a half past K): 16 bytes
  // (4-bit codes) in cw, 32 bytes (8-bit codes) in cw and cw2
  u32x4_t cw[NJ], cw2[CB == 8 ? NJ : 1];
  auto read_codes = [&](int kt, bool check_k) __attribute__((always_inline)) {
    const uint16_t* Cs = lds_code[(kt / kTilesPerGroup) & 1];
    if constexpr (CB == 4) {
      const int c = code_chunk(0, 2 * (kt % kTilesPerGroup) + fk) ^ code_x;
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        cw[j] = *reinterpret_cast<const u32x4_t*>(Cs + code_off0 + 32 * j * (kCodeRowBytes / 2) + 8 * c);
    } else {
      const int c0 = code_chunk(0, 4 * (kt % kTilesPerGroup) + 2 * fk) ^ code_x;
      const int c1 = code_chunk(0, 4 * (kt % kTilesPerGroup) + 2 * fk + 1) ^ code_x;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        cw[j] = *reinterpret_cast<const u32x4_t*>(Cs + code_off0 + 32 * j * (kCodeRowBytes / 2) + 8 * c0);
        cw2[j] = *reinterpret_cast<const u32x4_t*>(Cs + code_off0 + 32 * j * (kCodeRowBytes / 2) + 8 * c1);
      }
    }
    if (check_k && kt * BK + 32 * fk >= K) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        cw[j] = u32x4_t{0u, 0u, 0u, 0u};
        if constexpr (CB == 8) cw2[j] = u32x4_t{0u, 0u, 0u, 0u};
      }
    }
  };
  // zero the A chunks of the tile past K (the last tile only)
  auto zero_tail_a = [&](int kt, int sa) __attribute__((always_inline)) {
    uint16_t* As = stage_a(sa);
#pragma unroll
    for (int i = 0; i < RA; ++i) {
      const int row = SEG_ROWS * (NW * i + wv) + ld_sub;
      const int chunk = (swz<BK>(row, ld_phys) - row * BK) >> 3;
      if (kt * BK + 8 * chunk >= K)
        *reinterpret_cast<u32x4_t*>(As + (NW * i + wv) * 512 + 8 * lane) = u32x4_t{0u, 0u, 0u, 0u};
    }
  };

  f32x16_t acc[4][NJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  bf16x8_t fa[2][4];
  u32x4_t fbw[2][NJ];
  // A fragment of M block i, step s, from stage As
  auto load_fa = [&](const uint16_t* As, int s, int buf, int i) __attribute__((always_inline)) {
    fa[buf][i] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(As + swz<BK>(wm * 128 + 32 * i + fr, 4 * fk + s)));
  };
  // part p (2 codes -> 2 bf16) of B fragment j of step s; step 0 also marks
  // NaN blocks (one NaN element makes every output of the column NaN, as
  // the NaN weights would)
  auto cvt_part = [&](int s, int buf, int j, int p) __attribute__((always_inline)) {
    uint32_t v;
    if constexpr (FP4) {
      const uint32_t w = s == 0 ? cw[j].x : s == 1 ? cw[j].y : s == 2 ? cw[j].z : cw[j].w;
      if constexpr (NV) {
        const float sc = s >= 2 ? scf2[j] : scf[j];
        const f32x2v_t f = fp4_pair_f32(w, p);
        v = pack2(f.x * sc, f.y * sc);
      } else {
        v = cvt_fp4_pair(w, scf[j], p);
      }
      if (s == 0 && p == 0) v = (nan_j >> j) & 1 ? 0x7fc07fc0u : v;
    } else if constexpr (CB == 4) {
      // elements 2p, 2p + 1: the low and high nibble of byte p of word s,
      // i.e. byte p of the word's low and high nibbles spread to bytes
      // (the high nibbles stay in place, 16 times their value, and take
      // scale / 16; the masks are opaque so that each byte converts with
      // one v_cvt_f32_ubyte<p> instead of a field extract and a convert)
      const uint32_t w = s == 0 ? cw[j].x : s == 1 ? cw[j].y : s == 2 ? cw[j].z : cw[j].w;
      uint32_t lo, hi16;
      asm("v_and_b32 %0, 0x0f0f0f0f, %1" : "=v"(lo) : "v"(w));
      asm("v_and_b32 %0, 0xf0f0f0f0, %1" : "=v"(hi16) : "v"(w));
      v = pack2(fmaf(scf[j], ubyte(lo, p), sbi[j]), fmaf(scf[j] * 0.0625f, ubyte(hi16, p), sbi[j]));
    } else {
      // elements 2p, 2p + 1: bytes 2 (p % 2), +1 of word p / 2 of step s's 8 bytes
      const u32x4_t& c = s < 2 ? cw[j] : cw2[j];
      const uint32_t w = (s & 1) == 0 ? (p < 2 ? c.x : c.y) : (p < 2 ? c.z : c.w);
      v = pack2(fmaf(scf[j], ubyte(w, 2 * (p & 1)), sbi[j]), fmaf(scf[j], ubyte(w, 2 * (p & 1) + 1), sbi[j]));
    }
    if (p == 0) fbw[buf][j].x = v;
    else if (p == 1) fbw[buf][j].y = v;
    else if (p == 2) fbw[buf][j].z = v;
    else fbw[buf][j].w = v;
  };
  auto mfma_m = [&](int cur, int m) __attribute__((always_inline)) {
    const int i = m / NJ, j = m % NJ;
    acc[i][j] = mfma_32x32x16(fa[cur][i], __builtin_bit_cast(bf16x8_t, fbw[cur][j]), acc[i][j]);
  };

  // ---- prologue: A of tiles 0 and 1, code (and FAST: scale) groups 0 and 1,
  // (else: scales of tiles 0 and 1).  Tile kt uses A stage (kt + off) % 2;
  // FAST kernels pick off so that the last tile always uses stage 1 (every
  // step after the steady loop then has compile-time stages).
  const int off = FAST ? (ktiles & 1) : 0;
  issue_a(0, off);
  if (ktiles > 1) issue_a(1, off ^ 1);
  issue_codes(0);
  if (kCodeRowBytes < code_bytes) issue_codes(1);
  if constexpr (SCALE_LDS) {
    issue_scales(0);
    if (kCodeRowBytes < code_bytes) issue_scales(1);
    wait_vmcnt<0>();
    barrier_lds();
    load_scales(0);
    wait_lgkmcnt0();
    take_scales(0);
  } else {
    load_scales(0);
    wait_vmcnt<0>();
    take_scales(0);
    if (ktiles > 1) load_scales(1);
  }
  barrier_lds();
  if (tail_tile == 0) {
    zero_tail_a(0, 0);
    barrier_lds();
  }
  read_codes(0, true);
#pragma unroll
  for (int i = 0; i < 4; ++i) load_fa(stage_a(off), 0, 0, i);
  wait_lgkmcnt0();
#pragma unroll
  for (int m = 0; m < NM; ++m) cvt_part(0, 0, m / 4, m % 4);

  // One K tile.  Steps 0..2: the MFMAs of step s alternate with the A
  // fragment reads and B fragment conversions of step s + 1.  Step 3 starts
  // with the tile boundary (all copies landed, barrier: tile kt+1 is in LDS
  // and every wavefront is done reading tile kt), reads tile kt+1's codes and
  // scales, then alternates its MFMAs with the copies of A(kt+2) into the
  // stage tile kt used and with tile kt+1's first fragments.
  // MODE kSteady: tile kt+1 exists and is no tail tile (copies past the last
  // tile are clamped to it, into a stage nobody reads again); kFinal: tile
  // kt+1 is the last one (no copies); kLast: tile kt is the last one;
  // kGeneral: run-time checks.
  auto tile_step = [&](int kt, auto mode_tag, auto phase_tag) __attribute__((always_inline)) {
    constexpr int MODE = decltype(mode_tag)::value;
    constexpr bool STEADY = MODE == kSteady || MODE == kFinal;
    constexpr bool COPIES = MODE != kFinal;
    constexpr int PH = decltype(phase_tag)::value;  // kt % 2 if >= 0
    const int sa = PH >= 0 ? PH : kt & 1;
    const int sa1 = PH >= 0 ? PH ^ 1 : (kt + 1) & 1;
#pragma unroll
    for (int s = 0; s < KK; ++s) {
      const int cur = s & 1, nxt = cur ^ 1;
      wait_lgkmcnt0();
      if (s + 1 < KK) {
        const uint16_t* As = stage_a(sa);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          mfma_m(cur, m);
          if (m < 4) load_fa(As, s + 1, nxt, m);
          cvt_part(s + 1, nxt, m / 4, m % 4);
          __builtin_amdgcn_sched_barrier(0);
        }
        continue;
      }
      if (MODE == kLast || (MODE == kGeneral && kt + 1 >= ktiles)) {
#pragma unroll
        for (int m = 0; m < NM; ++m) mfma_m(cur, m);
        continue;
      }
      wait_vmcnt<0>();
      barrier_lds();
      if (!STEADY && kt + 1 == tail_tile) {
        zero_tail_a(kt + 1, sa1);
        barrier_lds();
      }
      read_codes(kt + 1, !STEADY);
      if constexpr (SCALE_LDS) {
        load_scales(kt + 1);  // LDS reads; converted once they have landed
      } else {
        take_scales(kt + 1);
        if (COPIES && (STEADY || kt + 2 < ktiles)) load_scales(kt + 2);
      }
      const int g1 = (kt + 1) / kTilesPerGroup + 1;
      if (COPIES && (kt + 1) % kTilesPerGroup == 0 && kCodeRowBytes * g1 < code_bytes) {
        issue_codes(g1);
        if constexpr (SCALE_LDS) issue_scales(g1);
      }
      const bool more_a = STEADY || kt + 2 < ktiles;
      const int kt2 = min(kt + 2, ktiles - 1);
      uint16_t* As = stage_a(sa);
      const uint16_t* As1 = stage_a(sa1);
      __builtin_amdgcn_sched_barrier(0);
      if (STEADY) {
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          mfma_m(cur, m);
          if (COPIES && m < RA) copy_a(kt2, As, m);
          if (m < 4) load_fa(As1, 0, nxt, m);
          if (m == NM / 2 - 1) {
            wait_lgkmcnt0();
            if constexpr (SCALE_LDS) take_scales(kt + 1);
          }
          if (m >= NM / 2) {
            cvt_part(0, nxt, (2 * (m - NM / 2)) / 4, (2 * (m - NM / 2)) % 4);
            cvt_part(0, nxt, (2 * (m - NM / 2) + 1) / 4, (2 * (m - NM / 2) + 1) % 4);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int m = NM; m < RA; ++m)
          if (COPIES) copy_a(kt2, As, m);
      } else {
        if (more_a) issue_a(kt + 2, sa);
#pragma unroll
        for (int i = 0; i < 4; ++i) load_fa(As1, 0, nxt, i);
#pragma unroll
        for (int m = 0; m < NM; ++m) mfma_m(cur, m);
        wait_lgkmcnt0();
        if constexpr (SCALE_LDS) take_scales(kt + 1);
#pragma unroll
        for (int m = 0; m < NM; ++m) cvt_part(0, nxt, m / 4, m % 4);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  int kt = 0;
  if constexpr (FAST) {
    // stages: tile kt in (kt + off) % 2, the last tile in stage 1.  An odd
    // ktiles starts with one steady step in stage 1; then steady pairs up
    // to tile ktiles - 3, the final boundary (tile ktiles - 2, stage 0) and
    // the last tile.
    if (off && ktiles >= 2) {
      tile_step(0, int_c<kSteady>{}, int_c<1>{});
      kt = 1;
    }
    for (; kt + 2 <= ktiles - 2; kt += 2) {
      tile_step(kt, int_c<kSteady>{}, int_c<0>{});
      tile_step(kt + 1, int_c<kSteady>{}, int_c<1>{});
    }
    if (ktiles >= 2) tile_step(ktiles - 2, int_c<kFinal>{}, int_c<0>{});
    tile_step(ktiles - 1, int_c<kLast>{}, int_c<1>{});
  } else {
    const int steady_end = ktiles - 2 - (tail_tile >= 0 ? 1 : 0);
    for (; kt + 2 <= steady_end; kt += 2) {
      tile_step(kt, int_c<kSteady>{}, int_c<0>{});
      tile_step(kt + 1, int_c<kSteady>{}, int_c<1>{});
    }
    for (; kt < ktiles; ++kt) tile_step(kt, int_c<kGeneral>{}, int_c<-1>{});
  }

  store_tile<GATED, NJ, WN>(a, acc, e, false, N, n0, r0, r_end, wm, wn, lane);
}

// The FAST kernel applies when K % 64 == 0 and the scale tensors (MXFP4:
// e8m0 [E, N, K / 32]; affine: bf16 scales and biases [E, N, K / G]) are
// 4-byte aligned in base and size: their dwords are then copied whole.
bool fast_shape(const Layer& L, int K, int N, const void* scales, const void* biases) {
  if (K % BK) return false;
  const bool mx = L.wfmt == WF_MXFP4 || L.wfmt == WF_NVFP4;  // byte scales, no biases
  const int group = L.wfmt == WF_AFF8 ? 64 : L.wfmt == WF_NVFP4 ? 16 : 32;
  const size_t bytes = (size_t)L.E * N * (K / group) * (mx ? 1 : 2);
  const auto aligned = [](const void* p) { return reinterpret_cast<uintptr_t>(p) % 4 == 0; };
  return bytes % 4 == 0 && aligned(scales) && (mx || aligned(biases));
}

template <int FMT, bool GATED, int NJ, int WN>
void launch_fmt(const MfmaArgs& m, dim3 grid, bool fast, hipStream_t s) {
  if (fast) lowbit_gemm_kernel<FMT, GATED, NJ, true, WN><<<grid, 128 * WN, 0, s>>>(m);
  else lowbit_gemm_kernel<FMT, GATED, NJ, false, WN><<<grid, 128 * WN, 0, s>>>(m);
}

// NJ = 32-column results per wavefront with WN = 2: 4 (256 columns a tile) or
// 3 (192).  MXFP4 256-column tiles may run as 8 wavefronts of 128 x 64.
template <bool GATED, int NJ>
void launch_any(const Layer& L, const MfmaArgs& m, dim3 grid, bool fast, hipStream_t s) {
  if (L.wfmt == WF_MXFP4) {
    if constexpr (NJ == 4 && kMx4WavesN == 4) launch_fmt<kFmtMx4, GATED, 2, 4>(m, grid, fast, s);
    else launch_fmt<kFmtMx4, GATED, NJ, 2>(m, grid, fast, s);
  } else if (L.wfmt == WF_NVFP4) {
    launch_fmt<kFmtNv4, GATED, NJ, 2>(m, grid, fast, s);
  } else if (L.wfmt == WF_AFF4) {
    launch_fmt<kFmtAff4, GATED, NJ, 2>(m, grid, fast, s);
  } else {
    launch_fmt<kFmtAff8, GATED, NJ, 2>(m, grid, fast, s);
  }
}

}  // namespace

hipError_t launch_gate_up_lowbit(const Layer& L, const Work& W, hipStream_t s) {
  MfmaArgs m = base_args(L, W);
  m.a = static_cast<const uint16_t*>(L.x);
  m.lda = L.d;
  m.row_token = W.row_token;
  m.c0 = L.wg_codes; m.s0 = L.wg_scales; m.c1 = L.wu_codes; m.s1 = L.wu_scales;
  m.qb0 = static_cast<const uint16_t*>(L.wg_qbias); m.qb1 = static_cast<const uint16_t*>(L.wu_qbias);
  m.ts0 = L.ts_g; m.ts1 = L.ts_u;
  m.bias0 = static_cast<const uint16_t*>(L.bg);
  m.bias1 = static_cast<const uint16_t*>(L.bu);
  m.N = L.F; m.K = L.d; m.N_sh = L.F; m.K_sh = L.d;
  m.out = static_cast<uint16_t*>(W.h);
  m.ldo = L.F_max();
  m.n_tiles = (L.F + 127) / 128;
  m.e_end = L.E;  // routed experts only: a shared expert's tiles go to the dense kernel
  const dim3 grid(grid_for(max_row_tiles(L, 0, L.E) * m.n_tiles));
  const bool fast = fast_shape(L, L.d, L.F, L.wg_scales, L.wg_qbias) && fast_shape(L, L.d, L.F, L.wu_scales, L.wu_qbias);
  launch_any<true, 4>(L, m, grid, fast, s);
  return hipGetLastError();
}

hipError_t launch_down_lowbit(const Layer& L, const Work& W, hipStream_t s) {
  MfmaArgs m = base_args(L, W);
  m.a = static_cast<const uint16_t*>(W.h);
  m.lda = L.F_max();
  m.row_token = nullptr;
  m.c0 = L.wd_codes; m.s0 = L.wd_scales;
  m.qb0 = static_cast<const uint16_t*>(L.wd_qbias);
  m.ts0 = L.ts_d;
  m.bias0 = static_cast<const uint16_t*>(L.bd);
  m.N = L.d; m.K = L.F; m.N_sh = L.d; m.K_sh = L.F;
  m.out = static_cast<uint16_t*>(W.y);
  m.ldo = L.d;
  // column tiles of 256 or 192, whichever copies fewer A bytes in total
  const int t192 = (L.d + 191) / 192, t256 = (L.d + 255) / 256;
  const bool narrow = t192 * (256 + 48) < t256 * (256 + 64);
  m.n_tiles = narrow ? t192 : t256;
  m.e_end = L.E;  // routed experts only: a shared expert's tiles go to the dense kernel
  const dim3 grid(grid_for(max_row_tiles(L, 0, L.E) * m.n_tiles));
  const bool fast = fast_shape(L, L.F, L.d, L.wd_scales, L.wd_qbias);
  if (narrow) launch_any<false, 3>(L, m, grid, fast, s);
  else launch_any<false, 4>(L, m, grid, fast, s);
  return hipGetLastError();
}

}  // namespace moe
