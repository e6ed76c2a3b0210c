// Expert stages for a few tokens (T <= 16): every expert holds at most 16
// sorted rows, so each stage is a stream over the active experts' weights.
//
//   gate|up:  h[r][f] = act(x[t] . Wg[e][f] + bg[e][f], x[t] . Wu[e][f] + bu[e][f])
//   down:     y[r][n] = h[r] . Wd[e][n] + bd[e][n]
//
// (MaxText GPT-OSS weight mapping "MOE EXPERTS"; glm4_moe_lite.go
// SwitchMLP.Forward and SharedExperts.Forward.)
//
// The stage is bound by HBM reads of the weights, and HBM streams fastest when
// every wavefront load instruction covers one contiguous kilobyte.  So the 64
// lanes of a wavefront split the reduction dimension of ONE weight row: lane l
// reads elements 512 c + 8 l .. +7 of chunk c, and multiplies them with the
// same elements of each of the expert's token rows (v_dot2_f32_bf16, fp32
// accumulation).  A wavefront owns kRowsPerWave consecutive weight rows (both
// the gate and the up row in the gated stage); one block of kWaves wavefronts
// owns kRowsPerWave * kWaves rows of one expert.  Blocks of experts without
// rows exit at once.
//
// MXFP4 weights (e2m1 codes, an e8m0 scale per 32): a lane takes blocks of
// 32 consecutive elements of a row, i.e. 16 bytes of codes under exactly one
// scale byte; v_cvt_scalef32_pk_bf16_fp4 turns each 8-element piece into bf16
// (exact: e2m1 times a power of two) for the same dot products.  A row is
// shared by 64, 32 or 16 lanes, whichever leaves the fewest idle lanes in a
// row's last step (decode_pass_fp4); a wavefront load then covers 1024, 512
// or 256 contiguous bytes of each of 1, 2 or 4 rows.
//
// After the reduction loop every lane holds partial sums of all
// (row, token) outputs; a reduce-scatter over the lanes of a row (halving the
// value set at each exchange step, DPP within 16 lanes, lane shuffles across)
// leaves each output summed over those lanes in one lane, in a fixed order,
// so the result does not depend on timing.
#include "device_common.h"
#include "moe_internal.h"

#ifndef MOE_DECODE_WAVES
#define MOE_DECODE_WAVES 4
#endif
// bf16: weight rows per wavefront and tokens per pass.  2 rows and passes of
// at most 8 tokens (113 registers: four wavefronts per SIMD in the gated stage)
// measured 0.7% faster per 8-token layer step than 4 rows and passes of 16.
#ifndef MOE_DECODE_ROWS
#define MOE_DECODE_ROWS 2
#endif
#ifndef MOE_DECODE_MAX_TG
#define MOE_DECODE_MAX_TG 8
#endif
// MXFP4: tokens per pass, and how many of a chunk's four 8-element pieces
// are unrolled (see the MXFP4 shapes below)
#ifndef MOE_DECODE_FP4_TG
#define MOE_DECODE_FP4_TG 2
#endif
#ifndef MOE_DECODE_FP4_UNROLL
#define MOE_DECODE_FP4_UNROLL 4
#endif

namespace moe {
namespace {

constexpr int kWaves = MOE_DECODE_WAVES;
constexpr int kRowsPerWave = MOE_DECODE_ROWS;
constexpr int kRowsPerBlock = kWaves * kRowsPerWave;
// Token rows handled in one pass over the weights (power of two).
constexpr int kMaxTg = MOE_DECODE_MAX_TG;
// Elements of a weight row covered by one wavefront load (64 lanes x 8).
constexpr int kChunk = 512;
static_assert((kRowsPerWave & (kRowsPerWave - 1)) == 0, "rows per wavefront must be a power of two");
static_assert(kMaxTg >= 1 && kMaxTg <= kDecodeMaxTokens && (kMaxTg & (kMaxTg - 1)) == 0, "bad token group");

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

struct DecodeArgs {
  const uint16_t* a;          // gate|up: x [T, lda]; down: h [rows, lda]
  int lda;
  const int32_t* row_token;   // gate|up: token of each sorted row; down: nullptr
  const uint16_t* w0;         // [E, N, K]: down, or gate
  const uint16_t* w1;         // up (gate|up only)
  const uint8_t* c0;          // MXFP4: codes [E, N, K / 2] and e8m0 scales [E, N, K / 32] of w0 / w1
  const uint8_t* s0;
  const uint8_t* c1;
  const uint8_t* s1;
  const uint16_t* bias0;      // [E, N] or nullptr
  const uint16_t* bias1;
  const uint16_t* sh_w0;      // shared expert [N_sh, K_sh] or nullptr
  const uint16_t* sh_w1;
  int N, K, N_sh, K_sh;
  int E;
  const int32_t* offsets;     // [E_all + 1]
  uint16_t* out;
  int ldo;
  int act;
  float alpha, limit;
};

__device__ __forceinline__ u32x4_t ld16(const uint16_t* p) { return *reinterpret_cast<const u32x4_t*>(p); }
__device__ __forceinline__ u32x4_t ld16_stream(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}

// acc + sum over 8 bf16 products, pairwise in element order.  The pairs are
// taken with shufflevector: a bit_cast of a subscripted vector element
// (bit_cast<bf16x2>(w[i]) in an unrolled loop) is folded by this hipcc to
// element 0 for every i.
__device__ __forceinline__ float dot8(u32x4_t w, u32x4_t x, float acc) {
  const bf16x8_t a = __builtin_bit_cast(bf16x8_t, w), b = __builtin_bit_cast(bf16x8_t, x);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 0, 1), __builtin_shufflevector(b, b, 0, 1), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 2, 3), __builtin_shufflevector(b, b, 2, 3), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 4, 5), __builtin_shufflevector(b, b, 4, 5), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 6, 7), __builtin_shufflevector(b, b, 6, 7), acc, false);
  return acc;
}

// Exchange step j of the reduce-scatter: the partner of lane l is
// l ^ {15, 7, 2, 1, 16, 32}[j] (row mirror, half-row mirror, quad swaps, then
// across 16- and 32-lane halves).  Each partner differs from l in the step's
// decision bit {3, 2, 1, 0, 4, 5}[j] and agrees on the earlier ones.
constexpr int kDecisionBit[6] = {3, 2, 1, 0, 4, 5};
template <int J>
__device__ __forceinline__ float exchange(float v) {
  const int i = __builtin_bit_cast(int, v);
  if constexpr (J == 0) return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(i, 0x140, 0xF, 0xF, true));
  else if constexpr (J == 1) return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(i, 0x141, 0xF, 0xF, true));
  else if constexpr (J == 2) return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(i, 0x4E, 0xF, 0xF, true));
  else if constexpr (J == 3) return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(i, 0xB1, 0xF, 0xF, true));
  else if constexpr (J == 4) return __shfl_xor(v, 16, 64);
  else return __shfl_xor(v, 32, 64);
}

// Reduce-scatter of v[0 .. C) over the wavefront.  While C > 1 a step keeps the
// half of the values selected by the lane's decision bit and adds the
// partner's copy of that half; once one value is left the remaining steps add
// the partner's value.  Afterwards v[0 .. max(C/64, 1)) hold whole-wavefront
// sums (see lane_bits).  With JN < 6 only the first JN steps run: the sums are
// then over the lanes that agree in the remaining bits (lane bit 5 for JN = 5,
// bits 4 and 5 for JN = 4), i.e. over each 32- or 16-lane group.
template <int J, int C, int JN = 6>
__device__ __forceinline__ void reduce_scatter(float* v, int lane) {
  if constexpr (J < JN) {
    const bool hi = (lane >> kDecisionBit[J]) & 1;
    if constexpr (C > 1) {
      constexpr int H = C / 2;
#pragma unroll
      for (int i = 0; i < H; ++i) {
        const float keep = hi ? v[H + i] : v[i];
        const float send = hi ? v[i] : v[H + i];
        v[i] = keep + exchange<J>(send);
      }
      reduce_scatter<J + 1, H, JN>(v, lane);
    } else {
      v[0] += exchange<J>(v[0]);
      reduce_scatter<J + 1, 1, JN>(v, lane);
    }
  }
}

constexpr int ilog2(int v) { return v <= 1 ? 0 : 1 + ilog2(v / 2); }

// After reduce_scatter of V values (JN steps), lane `lane` holds in v[i] the
// value with index lane_bits * max(V/2^JN, 1) + i, where lane_bits collects the
// decision bits of the first min(log2 V, JN) steps, most significant first.
// Lanes that differ only in the other decision bits of those JN steps hold the
// same sums; the one with those bits zero is the owner.
template <int V, int JN = 6>
__device__ __forceinline__ int lane_bits(int lane) {
  constexpr int S = ilog2(V) < JN ? ilog2(V) : JN;
  int b = 0;
#pragma unroll
  for (int j = 0; j < S; ++j) b = (b << 1) | ((lane >> kDecisionBit[j]) & 1);
  return b;
}
template <int V, int JN = 6>
__device__ __forceinline__ bool lane_owns(int lane) {
  constexpr int S = ilog2(V) < JN ? ilog2(V) : JN;
  bool own = true;
#pragma unroll
  for (int j = S; j < JN; ++j) own = own && !((lane >> kDecisionBit[j]) & 1);
  return own;
}

// e8m0 scale byte as the fp32 factor of the conversion (0: 2^-127, a
// denormal; 255, NaN, is marked by the caller)
__device__ __forceinline__ float e8m0_factor(uint32_t s) { return __uint_as_float(s == 0 ? 0x00400000u : (s << 23)); }

// Word q of 16 bytes of e2m1 codes (8 codes, low nibble first) times the
// scale as 8 bf16, in element order.
__device__ __forceinline__ u32x4_t fp4_word_bf16(uint32_t w, float scale) {
  u32x4_t r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0));
  r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1));
  r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2));
  r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3));
  return r;
}

// Bias, activation and bf16 store of a pass's outputs after the reduction.
// Value index ((g S + s) TG + t): tensor g (gate 0, up 1), row slot s, token
// slot t.  Row slot s of the wavefront covers rows nw + s RPS + (0 .. RPS-1),
// one per group of LPR lanes (lane / LPR picks the row; RPS = 64 / LPR).
template <bool GATED, int TG, int S, int LPR>
__device__ __forceinline__ void store_pass(const DecodeArgs& a, float* v, int e, bool shared, int N, int nw, int m0,
                                           int m, int t0, int lane) {
  constexpr int G = GATED ? 2 : 1;
  constexpr int V = G * S * TG;
  constexpr int JN = ilog2(LPR);
  constexpr int RPS = 64 / LPR;
  reduce_scatter<0, V, JN>(v, lane);

  constexpr int C = V >= LPR ? V / LPR : 1;
  const int lb = lane_bits<V, JN>(lane);
  const bool own = lane_owns<V, JN>(lane);
  const int sub = lane / LPR;
#pragma unroll
  for (int i = 0; i < C; ++i) {
    // the gate/up index bit is the most significant, taken from lane bit 3:
    // the up value of a gate lane sits in lane ^ 8 (row rotate by 8)
    float up = 0.f;
    if constexpr (GATED)
      up = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v[i]), 0x128, 0xF, 0xF, true));
    const int idx = lb * C + i;
    const int g = idx / (S * TG), s = (idx / TG) % S, t = idx % TG;
    const int n = nw + s * RPS + sub;
    if (!own || g != 0 || t0 + t >= m || n >= N) continue;
    float val = v[i];
    if (!shared && a.bias0) val += bf16_to_f32(a.bias0[(size_t)e * N + n]);
    if constexpr (GATED) {
      if (!shared && a.bias1) up += bf16_to_f32(a.bias1[(size_t)e * N + n]);
      val = expert_act(shared ? 1 : a.act, val, up, a.alpha, a.limit);
    }
    a.out[(size_t)(m0 + t0 + t) * a.ldo + n] = f32_to_bf16(val);
  }
}

// Token rows t0 .. t0+TG-1 of the expert (slots >= m repeat slot m - 1; they
// contribute zeros and are not stored).
template <int TG>
__device__ __forceinline__ void token_rows(const DecodeArgs& a, int m0, int m, int t0, const uint16_t* (&X)[TG]) {
#pragma unroll
  for (int t = 0; t < TG; ++t) {
    const int slot = min(t0 + t, m - 1);
    const int brow = a.row_token ? a.row_token[m0 + slot] : m0 + slot;
    X[t] = a.a + (size_t)brow * a.lda;
  }
}

// One pass over the wavefront's R bf16 weight rows for token slots
// t0 .. t0+TG-1 of the expert.
template <bool GATED, int TG, int R>
__device__ __forceinline__ void decode_pass(const DecodeArgs& a, int e, bool shared, int N, int K, int nw, int m0,
                                            int m, int t0, int lane) {
  constexpr int G = GATED ? 2 : 1;
  constexpr int V = G * R * TG;  // value index ((g R + r) TG + t)
  static_assert((V & (V - 1)) == 0, "value count must be a power of two");

  const uint16_t* Wb0 = shared ? a.sh_w0 : a.w0 + (size_t)e * a.N * a.K;
  const uint16_t* Wb1 = GATED ? (shared ? a.sh_w1 : a.w1 + (size_t)e * a.N * a.K) : nullptr;
  const uint16_t* Wr[G][R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const size_t row = (size_t)min(nw + r, N - 1) * K;  // rows past N are computed but not stored
    Wr[0][r] = Wb0 + row;
    if constexpr (GATED) Wr[1][r] = Wb1 + row;
  }
  const uint16_t* X[TG];
  token_rows<TG>(a, m0, m, t0, X);

  float v[V];
#pragma unroll
  for (int i = 0; i < V; ++i) v[i] = 0.f;

  const int chunks = (K + kChunk - 1) / kChunk;
  for (int c = 0; c < chunks; ++c) {
    const int k = c * kChunk + 8 * lane;
    if (k < K) {  // K % 8 == 0: a lane's 8 elements are all in range or all out
      u32x4_t w[G][R], x[TG];
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int r = 0; r < R; ++r) w[g][r] = ld16_stream(Wr[g][r] + k);
#pragma unroll
      for (int t = 0; t < TG; ++t) x[t] = (t0 + t < m) ? ld16(X[t] + k) : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int t = 0; t < TG; ++t) v[(g * R + r) * TG + t] = dot8(w[g][r], x[t], v[(g * R + r) * TG + t]);
    }
  }
  store_pass<GATED, TG, R, 64>(a, v, e, shared, N, nw, m0, m, t0, lane);
}

// One pass over the wavefront's R MXFP4 weight rows.  A row of K elements is
// KB = K / 32 blocks, each 16 bytes of codes under one scale byte.  LPR lanes
// share a row: lane l takes blocks l % LPR + LPR j (j = 0, 1, ...) of row
// l / LPR of each slot of RPS = 64 / LPR consecutive rows.  A 64-lane row
// step wastes the lanes past KB in its last step (K = 2880: 90 blocks in two
// steps of 64, 26 lanes busy in the second); 32 lanes per row cover two rows
// in three steps of 32 blocks each, i.e. 1.5 full-wavefront steps per row
// instead of 2, and a load instruction covers 512 contiguous bytes of each of
// the two rows.  Measured on the 8-token layer (K = 2880): gate|up 57.0 ->
// 50.4 us, and with 8 down rows per wavefront the step 0.1003 -> 0.0915 ms.
template <bool GATED, int TG, int R, int LPR>
__device__ __forceinline__ void decode_pass_fp4(const DecodeArgs& a, int e, bool shared, int N, int K, int nw, int m0,
                                                int m, int t0, int lane) {
  constexpr int G = GATED ? 2 : 1;
  constexpr int RPS = 64 / LPR;
  static_assert(R % RPS == 0, "rows per wavefront must fill its row slots");
  constexpr int S = R / RPS;
  constexpr int V = G * S * TG;  // value index ((g S + s) TG + t)
  static_assert((V & (V - 1)) == 0, "value count must be a power of two");

  const uint16_t* X[TG];
  token_rows<TG>(a, m0, m, t0, X);
  const int sub = lane / LPR, pos = lane % LPR;
  // codes and scales of the lane's row in each slot (rows past N read row N - 1)
  const uint8_t* Cr[G][S];
  const uint8_t* Sr[G][S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const size_t row = (size_t)e * N + min(nw + s * RPS + sub, N - 1);
    Cr[0][s] = a.c0 + row * (K / 2);
    Sr[0][s] = a.s0 + row * (K / 32);
    if constexpr (GATED) {
      Cr[1][s] = a.c1 + row * (K / 2);
      Sr[1][s] = a.s1 + row * (K / 32);
    }
  }

  float v[V];
#pragma unroll
  for (int i = 0; i < V; ++i) v[i] = 0.f;

  const int KB = K / 32;
  const int steps = (KB + LPR - 1) / LPR;
  for (int j = 0; j < steps; ++j) {
    const int kb = pos + LPR * j;
    if (kb < KB) {
      const int k = 32 * kb;
      u32x4_t wc[G][S];
      float sf[G][S];
      bool nan[G][S];
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int s = 0; s < S; ++s) {
          wc[g][s] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(Cr[g][s] + 16 * kb));
          const uint32_t sb = Sr[g][s][kb];
          sf[g][s] = e8m0_factor(sb);
          nan[g][s] = sb == 255u;
        }
      // the four 8-element pieces, unrolled: each piece's code word is then
      // picked at compile time (a rolled loop selects it with three
      // v_cndmask per word and row), at the price of every token's 32
      // elements held at once
#pragma unroll MOE_DECODE_FP4_UNROLL
      for (int q = 0; q < 4; ++q) {
        u32x4_t x[TG];
#pragma unroll
        for (int t = 0; t < TG; ++t) x[t] = (t0 + t < m) ? ld16(X[t] + k + 8 * q) : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int s = 0; s < S; ++s) {
            const uint32_t word = q == 0 ? wc[g][s].x : q == 1 ? wc[g][s].y : q == 2 ? wc[g][s].z : wc[g][s].w;
            u32x4_t w8 = fp4_word_bf16(word, sf[g][s]);
            // a NaN block: one NaN weight makes the row's sums NaN, as the oracle's would be
            if (q == 0 && nan[g][s]) w8.x = 0x7fc07fc0u;
#pragma unroll
            for (int t = 0; t < TG; ++t) v[(g * S + s) * TG + t] = dot8(w8, x[t], v[(g * S + s) * TG + t]);
          }
      }
    }
  }
  store_pass<GATED, TG, S, LPR>(a, v, e, shared, N, nw, m0, m, t0, lane);
}

// MXFP4 shapes.  The conversions and dot products of 4.25-bit weights cost
// more issue slots per byte than the loads, so the shapes minimise vector
// instructions per weight: a pass takes at most 2 tokens (the widest token
// group sets the register budget of the whole kernel, and an expert with more
// rows makes more passes over its weights), a wavefront takes 4 rows of gate
// and up or 8 rows of down, and the lanes per row are chosen per launch from
// K.  Measured on the 8-token layer (64 lanes per row then) against 4 tokens,
// rolled pieces and 8 down rows: gate|up 69.2 -> 57.7 us.  With 32 lanes per
// row: 8 gate|up rows 54.3 us against 50.4 for 4; 16 down rows 0.0947 ms per
// step against 0.0915 for 8; passes of 4 tokens 51.4 us.
#ifndef MOE_DECODE_FP4_RG
#define MOE_DECODE_FP4_RG 4
#endif
#ifndef MOE_DECODE_FP4_RD
#define MOE_DECODE_FP4_RD 8
#endif
// Narrowest row share considered.  16 lanes per row (a load covering 256
// bytes of each of 4 rows) measured 18% slower on the gate|up rows of 2880
// than 32 lanes at the same lane count per row, so 16 is not taken by default.
#ifndef MOE_DECODE_FP4_MIN_LPR
#define MOE_DECODE_FP4_MIN_LPR 32
#endif
#ifndef MOE_DECODE_FP4_TIE_NARROW
#define MOE_DECODE_FP4_TIE_NARROW 0
#endif
constexpr int kFp4RowsGated = MOE_DECODE_FP4_RG, kFp4RowsDown = MOE_DECODE_FP4_RD, kFp4MaxTg = MOE_DECODE_FP4_TG;
template <bool GATED, bool FP4> constexpr int rows_per_wave() {
  return !FP4 ? kRowsPerWave : GATED ? kFp4RowsGated : kFp4RowsDown;
}
template <bool GATED, bool FP4> constexpr int max_token_group() { return FP4 ? kFp4MaxTg : kMaxTg; }

template <bool GATED, int TG, bool FP4, int R, int LPR>
__device__ __forceinline__ void run_pass(const DecodeArgs& a, int e, bool shared, int N, int K, int nw, int m0, int m,
                                         int t0, int lane) {
  if constexpr (FP4) decode_pass_fp4<GATED, TG, R, LPR>(a, e, shared, N, K, nw, m0, m, t0, lane);
  else decode_pass<GATED, TG, R>(a, e, shared, N, K, nw, m0, m, t0, lane);
}

// LPR: lanes per MXFP4 row (64 for bf16 weights)
template <bool GATED, bool FP4, int LPR = 64>
__global__ __launch_bounds__(64 * kWaves) void decode_kernel(DecodeArgs a) {
  constexpr int RW = rows_per_wave<GATED, FP4>();
  const int e = blockIdx.y;
  const bool shared = e >= a.E;
  const int N = shared ? a.N_sh : a.N;
  const int K = shared ? a.K_sh : a.K;
  const int nb = blockIdx.x * RW * kWaves;
  if (nb >= N) return;
  const int m0 = a.offsets[e];
  const int m = a.offsets[e + 1] - m0;  // <= kDecodeMaxTokens on this path
  if (m <= 0) return;
  const int lane = threadIdx.x & 63;
  const int nw = nb + (threadIdx.x >> 6) * RW;
  if (nw >= N) return;
  // token group: the smallest power of two covering m, up to MT per pass
  constexpr int MT = max_token_group<GATED, FP4>();
  if (m <= 1) {
    run_pass<GATED, 1, FP4, RW, LPR>(a, e, shared, N, K, nw, m0, m, 0, lane);
  } else if (m <= 2) {
    run_pass<GATED, 2, FP4, RW, LPR>(a, e, shared, N, K, nw, m0, m, 0, lane);
  } else if (m <= 4 || MT < 8) {
    for (int t0 = 0; t0 < m; t0 += 4 < MT ? 4 : MT)
      run_pass<GATED, (4 < MT ? 4 : MT), FP4, RW, LPR>(a, e, shared, N, K, nw, m0, m, t0, lane);
  } else if (m <= 8 || MT < 16) {
    for (int t0 = 0; t0 < m; t0 += 8) run_pass<GATED, 8, FP4, RW, LPR>(a, e, shared, N, K, nw, m0, m, t0, lane);
  } else {
    run_pass<GATED, (MT < 16 ? 8 : 16), FP4, RW, LPR>(a, e, shared, N, K, nw, m0, m, 0, lane);
  }
}

// Lanes per MXFP4 row of K elements: the choice with the fewest lane-blocks
// per row, ceil(KB / LPR) LPR with KB = K / 32, the widest on a tie (longer
// contiguous loads, fewer token loads).  K = 2880: 32; K = 2048: 64.
int fp4_lanes_per_row(int K) {
  const int kb = K / 32;
  int best = 64, cost = (kb + 63) / 64 * 64;
  for (int lpr = 32; lpr >= MOE_DECODE_FP4_MIN_LPR; lpr /= 2) {
    const int c = (kb + lpr - 1) / lpr * lpr;
    if (c < cost || (MOE_DECODE_FP4_TIE_NARROW && c == cost)) {
      best = lpr;
      cost = c;
    }
  }
  return best;
}

template <bool GATED>
void launch_fp4(const DecodeArgs& d, int rows, int K, int n_experts, hipStream_t s) {
  constexpr int rb = rows_per_wave<GATED, true>() * kWaves;
  const dim3 grid((rows + rb - 1) / rb, n_experts);
  const int lpr = fp4_lanes_per_row(K);
  if constexpr (MOE_DECODE_FP4_MIN_LPR <= 16) {
    if (lpr == 16) return (void)decode_kernel<GATED, true, 16><<<grid, 64 * kWaves, 0, s>>>(d);
  }
  if constexpr (MOE_DECODE_FP4_MIN_LPR <= 32) {
    if (lpr == 32) return (void)decode_kernel<GATED, true, 32><<<grid, 64 * kWaves, 0, s>>>(d);
  }
  decode_kernel<GATED, true, 64><<<grid, 64 * kWaves, 0, s>>>(d);
}

DecodeArgs base_args(const Layer& L, const Work& W) {
  DecodeArgs d{};
  d.E = L.E;
  d.offsets = W.offsets;
  d.act = L.act;
  d.alpha = L.alpha;
  d.limit = L.limit;
  return d;
}

}  // namespace

hipError_t launch_gate_up_decode(const Layer& L, const Work& W, hipStream_t s) {
  DecodeArgs d = base_args(L, W);
  d.a = static_cast<const uint16_t*>(L.x);
  d.lda = L.d;
  d.row_token = W.row_token;
  d.w0 = static_cast<const uint16_t*>(L.wg);
  d.w1 = static_cast<const uint16_t*>(L.wu);
  d.bias0 = static_cast<const uint16_t*>(L.bg);
  d.bias1 = static_cast<const uint16_t*>(L.bu);
  d.sh_w0 = static_cast<const uint16_t*>(L.sh_wg);
  d.sh_w1 = static_cast<const uint16_t*>(L.sh_wu);
  d.c0 = L.wg_codes; d.s0 = L.wg_scales; d.c1 = L.wu_codes; d.s1 = L.wu_scales;
  d.N = L.F; d.K = L.d; d.N_sh = L.F_sh; d.K_sh = L.d;
  d.out = static_cast<uint16_t*>(W.h);
  d.ldo = L.F_max();
  if (L.wfmt == WF_MXFP4) {
    launch_fp4<true>(d, L.F_max(), L.d, L.n_experts_all(), s);
  } else {
    const dim3 grid((L.F_max() + kRowsPerBlock - 1) / kRowsPerBlock, L.n_experts_all());
    decode_kernel<true, false><<<grid, 64 * kWaves, 0, s>>>(d);
  }
  return hipGetLastError();
}

hipError_t launch_down_decode(const Layer& L, const Work& W, hipStream_t s) {
  DecodeArgs d = base_args(L, W);
  d.a = static_cast<const uint16_t*>(W.h);
  d.lda = L.F_max();
  d.row_token = nullptr;
  d.w0 = static_cast<const uint16_t*>(L.wd);
  d.bias0 = static_cast<const uint16_t*>(L.bd);
  d.sh_w0 = static_cast<const uint16_t*>(L.sh_wd);
  d.c0 = L.wd_codes; d.s0 = L.wd_scales;
  d.N = L.d; d.K = L.F; d.N_sh = L.d; d.K_sh = L.F_sh;
  d.out = static_cast<uint16_t*>(W.y);
  d.ldo = L.d;
  if (L.wfmt == WF_MXFP4) {
    launch_fp4<false>(d, L.d, L.F, L.n_experts_all(), s);
  } else {
    const dim3 grid((L.d + kRowsPerBlock - 1) / kRowsPerBlock, L.n_experts_all());
    decode_kernel<false, false><<<grid, 64 * kWaves, 0, s>>>(d);
  }
  return hipGetLastError();
}

}  // namespace moe
