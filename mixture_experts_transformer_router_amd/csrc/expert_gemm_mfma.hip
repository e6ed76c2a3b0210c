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
// Block tile 256 rows x 256 columns, K staged 64 at a time through two LDS
// buffers: the copies of tile k+1 (global -> LDS directly, no registers) are
// in flight while tile k is multiplied.
// 4 wavefronts, each owning a 128 x 128 sub-tile as 4 x 4 results of
// v_mfma_f32_32x32x16_bf16 (fp32 accumulators).  LDS rows are 128 bytes (64
// bf16); the 16-byte chunk c of row r is stored at chunk c ^ (r & 7), so the
// 16-byte fragment reads of 8 consecutive rows hit 8 different bank groups.
//
// gate|up: the block's 256 columns are 128 gate and the same 128 up rows of
// the expert, interleaved by 32 (gate, up, gate, up within each wavefront), so
// one lane holds g and u of the same (row, f) and the activation is applied
// in registers.  Token rows are gathered while loading (no permuted copy of
// x).  MXFP4 weights: the loader decodes e2m1 codes with their e8m0 block
// scale to bf16 in LDS (exact: every value is a bf16 number).
#include "device_common.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int BM = kTileMBig;  // 256
constexpr int BN = 256;
constexpr int BK = 64;
constexpr int kThreads = 256;

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
  int n_tiles;                // column tiles per row tile
  uint16_t* out;
  int ldo;
  int act;
  float alpha, limit;
};

__device__ __forceinline__ int swz(int row, int chunk) { return row * BK + ((chunk ^ (row & 7)) << 3); }

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

template <int WF, bool GATED>
__global__ __launch_bounds__(kThreads, 1) void mfma_gemm_kernel(MfmaArgs a) {
  __shared__ uint16_t lds[2][2][BM * BK];  // [stage][A | B] -- 128 KB

  const int m_tile = blockIdx.x / a.n_tiles;
  const int n_tile = blockIdx.x % a.n_tiles;
  if (m_tile >= a.tile_prefix[a.E_all]) return;
  int lo = 0, hi = a.E_all - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.tile_prefix[mid] <= m_tile) lo = mid; else hi = mid - 1;
  }
  const int e = lo;
  const bool shared = e >= a.E;
  const int N = shared ? a.N_sh : a.N;
  const int K = shared ? a.K_sh : a.K;
  const int n0 = n_tile * (GATED ? BN / 2 : BN);
  if (n0 >= N) return;
  const int r0 = a.offsets[e] + (m_tile - a.tile_prefix[e]) * BM;
  const int r_end = a.offsets[e + 1];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv >> 1, wn = wv & 1;

  // ---- loaders.  Global -> LDS copies go straight into LDS (16 bytes per
  // lane): in round i, wavefront wv fills LDS rows 8 (4 i + wv) .. +7, lane l
  // the 16-byte slot l of that 1 KB segment, i.e. row 8 (4 i + wv) + (l >> 3),
  // stored chunk l & 7, which holds logical chunk (l & 7) ^ (row & 7).
  // Rows past the expert's last row (A) or past N (B) load a valid row
  // instead: they only feed outputs that the epilogue drops.  Chunks past K
  // are zero-filled with an ordinary LDS store.
  const int ld_sub = lane >> 3;                          // row within the segment
  const int ld_chunk = (lane & 7) ^ (ld_sub & 7);        // logical chunk loaded
  int a_row[8];
  int b_row[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = 8 * (4 * i + wv) + ld_sub;
    const int gr = r0 + r < r_end ? r0 + r : r0;
    a_row[i] = a.row_token ? a.row_token[gr] : gr;
    if constexpr (WF != WF_MXFP4) {
      // B row r of the tile -> weight row of the expert (-1: the up matrix, encoded below)
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
  }
  const uint16_t* w_gate = shared ? a.sh_w0 : a.w0 + (size_t)e * a.N * K;
  const uint16_t* w_up = GATED ? (shared ? a.sh_w1 : a.w1 + (size_t)e * a.N * K) : nullptr;

  // MXFP4: thread t decodes B row t (64 elements per K tile) through registers
  const uint8_t* mx_codes = nullptr;
  const uint8_t* mx_scales = nullptr;
  if constexpr (WF == WF_MXFP4) {
    const int r = tid;
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
  u32x4_t mxr[3];

  // full K tiles (tail == false) need no bounds checks
  auto issue_tile = [&](int k0, int stage, bool tail) {
    const int k = k0 + 8 * ld_chunk;
    const bool k_ok = !tail || k < K;
    uint16_t* As = lds[stage][0];
    uint16_t* Bs = lds[stage][1];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint16_t* seg = As + (4 * i + wv) * 512;  // 1 KB segment (512 bf16)
      if (k_ok) {
        __builtin_amdgcn_global_load_lds(a.a + (size_t)a_row[i] * a.lda + k, seg, 16, 0, 0);
      } else {
        *reinterpret_cast<u32x4_t*>(seg + 8 * lane) = u32x4_t{0u, 0u, 0u, 0u};
      }
    }
    if constexpr (WF == WF_MXFP4) {
      const bool ok0 = mx_codes && k0 < K, ok1 = mx_codes && k0 + 32 < K;
      mxr[0] = ok0 ? *reinterpret_cast<const u32x4_t*>(mx_codes + k0 / 2) : u32x4_t{0u, 0u, 0u, 0u};
      mxr[1] = ok1 ? *reinterpret_cast<const u32x4_t*>(mx_codes + k0 / 2 + 16) : u32x4_t{0u, 0u, 0u, 0u};
      mxr[2] = u32x4_t{ok0 ? (uint32_t)mx_scales[k0 / 32] : 127u, ok1 ? (uint32_t)mx_scales[k0 / 32 + 1] : 127u, 0u, 0u};
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        uint16_t* seg = Bs + (4 * i + wv) * 512;
        if (k_ok) {
          const uint16_t* wsrc = (b_row[i] & 1) ? w_up : w_gate;
          __builtin_amdgcn_global_load_lds(wsrc + (size_t)(b_row[i] >> 1) * K + k, seg, 16, 0, 0);
        } else {
          *reinterpret_cast<u32x4_t*>(seg + 8 * lane) = u32x4_t{0u, 0u, 0u, 0u};
        }
      }
    }
  };
  // MXFP4 only: decode the staged codes of row tid into LDS
  auto finish_tile = [&](int stage) {
    if constexpr (WF == WF_MXFP4) {
      uint16_t* Bs = lds[stage][1];
#pragma unroll
      for (int c = 0; c < 8; ++c)
        *reinterpret_cast<u32x4_t*>(Bs + swz(tid, c)) = decode_e2m1x8(mxr[c >> 2][c & 3], mxr[2][c >> 2]);
    }
  };

  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  const int ktiles = (K + BK - 1) / BK;
  const int full_tiles = K / BK;  // tiles with no element past K
  issue_tile(0, 0, full_tiles == 0);
  finish_tile(0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const int fr = lane & 31, fk = lane >> 5;
  for (int kt = 0; kt < ktiles; ++kt) {
    const int st = kt & 1;
    if (kt + 1 < full_tiles) issue_tile((kt + 1) * BK, st ^ 1, false);
    else if (kt + 1 < ktiles) issue_tile((kt + 1) * BK, st ^ 1, true);
    const uint16_t* As = lds[st][0];
    const uint16_t* Bs = lds[st][1];
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8_t af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(As + swz(wm * 128 + 32 * i + fr, 2 * kk + fk)));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bfr[j] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(Bs + swz(wn * 128 + 32 * j + fr, 2 * kk + fk)));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma_32x32x16(af[i], bfr[j], acc[i][j]);
    }
    if (kt + 1 < ktiles) finish_tile(st ^ 1);
    __builtin_amdgcn_s_waitcnt(0);  // this wavefront's LDS copies have landed
    __syncthreads();
  }

  // ---- epilogue: bias (+ activation) in registers, bf16 tile staged in LDS,
  // then written out as 16-byte row chunks.
  constexpr int OC = GATED ? BN / 2 : BN;     // output columns of the tile
  constexpr int OLD = GATED ? OC + 8 : OC;    // LDS row pitch (bf16); padded where it fits
  static_assert(BM * OLD * 2 <= (int)sizeof(lds), "output tile exceeds the LDS buffers");
  uint16_t* ot = &lds[0][0][0];
  const uint16_t* bias0 = shared ? nullptr : a.bias0;
  const uint16_t* bias1 = shared ? nullptr : a.bias1;
  const int act = shared ? 1 : a.act;
  if constexpr (GATED) {
    float bg[2], bu[2];
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int f = n0 + 32 * (2 * wn + jj) + fr;
      bg[jj] = (bias0 && f < N) ? bf16_to_f32(bias0[(size_t)e * N + f]) : 0.f;
      bu[jj] = (bias1 && f < N) ? bf16_to_f32(bias1[(size_t)e * N + f]) : 0.f;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int row = wm * 128 + 32 * i + 8 * (q >> 2) + 4 * fk + (q & 3);
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const float h = expert_act(act, acc[i][2 * jj][q] + bg[jj], acc[i][2 * jj + 1][q] + bu[jj], a.alpha, a.limit);
          ot[row * OLD + 32 * (2 * wn + jj) + fr] = f32_to_bf16(h);
        }
      }
  } else {
    float bv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + wn * 128 + 32 * j + fr;
      bv[j] = (bias0 && n < N) ? bf16_to_f32(bias0[(size_t)e * N + n]) : 0.f;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int row = wm * 128 + 32 * i + 8 * (q >> 2) + 4 * fk + (q & 3);
#pragma unroll
        for (int j = 0; j < 4; ++j) ot[row * OLD + wn * 128 + 32 * j + fr] = f32_to_bf16(acc[i][j][q] + bv[j]);
      }
  }
  __syncthreads();
  constexpr int CPR = OC / 8;  // 16-byte chunks per row
  const int rows = min(BM, r_end - r0);
  const int cols = min(OC, N - n0);  // multiple of 8
  for (int c = tid; c < BM * CPR; c += kThreads) {
    const int row = c / CPR, ch = c % CPR;
    if (row < rows && 8 * ch < cols) {
      u32x4_t v;
      const uint32_t* src = reinterpret_cast<const uint32_t*>(ot + row * OLD + 8 * ch);
      v[0] = src[0]; v[1] = src[1]; v[2] = src[2]; v[3] = src[3];
      *reinterpret_cast<u32x4_t*>(a.out + (size_t)(r0 + row) * a.ldo + n0 + 8 * ch) = v;
    }
  }
}

MfmaArgs base_args(const Layer& L, const Work& W) {
  MfmaArgs m{};
  m.E = L.E;
  m.E_all = L.n_experts_all();
  m.offsets = W.offsets;
  m.tile_prefix = W.tile_prefix_big;
  m.act = L.act;
  m.alpha = L.alpha;
  m.limit = L.limit;
  return m;
}

int max_row_tiles(const Layer& L) { return (L.rows_all() + BM - 1) / BM + L.n_experts_all(); }

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
  m.n_tiles = (L.F_max() + BN / 2 - 1) / (BN / 2);
  const dim3 grid(max_row_tiles(L) * m.n_tiles);
  if (L.wfmt == WF_MXFP4) mfma_gemm_kernel<WF_MXFP4, true><<<grid, kThreads, 0, s>>>(m);
  else mfma_gemm_kernel<WF_BF16, true><<<grid, kThreads, 0, s>>>(m);
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
  m.n_tiles = (L.d + BN - 1) / BN;
  const dim3 grid(max_row_tiles(L) * m.n_tiles);
  if (L.wfmt == WF_MXFP4) mfma_gemm_kernel<WF_MXFP4, false><<<grid, kThreads, 0, s>>>(m);
  else mfma_gemm_kernel<WF_BF16, false><<<grid, kThreads, 0, s>>>(m);
  return hipGetLastError();
}

}  // namespace moe
