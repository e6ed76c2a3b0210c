// Grouped expert GEMMs on the vector ALUs for fp32 layers (fp32 data,
// fp32 accumulation):
//
//   gate|up:  for sorted row r of expert e with token t = row_token[r]
//             g = x[t] . Wg[e][f] + bg[e][f],  u = x[t] . Wu[e][f] + bu[e][f],
//             h[r][f] = act(g, u)
//   down:     y[r][n] = h[r] . Wd[e][n] + bd[e][n]
//
// (MaxText GPT-OSS weight mapping, "MOE EXPERTS": separate gate/up kernels and
// biases, down weight and bias; glm4_moe_lite.go SwitchMLP.Forward: gathered
// gate and up products, activation, gathered down product.)
//
// Tiling: a block owns a 64-row M-tile of one expert and 64 output columns
// (for gate|up: 64 gate and the same 64 up columns, so the activation is
// local).  256 threads; thread (ty, tx) accumulates rows ty + 16 i and columns
// tx + 16 j (i, j < 4) in fp32 over K chunks of 16 staged in LDS.  The M-tiles
// of all experts are numbered consecutively (tile_prefix); blocks past the
// last tile exit.  The shared expert, when present, is expert E with its own
// weights, no bias and the SiLU gate.
#include "device_common.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int BM = kTileM;  // 64
constexpr int BN = 64;
constexpr int BK = 16;

struct GemmArgs {
  const void* a;             // gate|up: x [T, K]; down: h [rows, lda]
  int lda;
  const int32_t* row_token;  // gate|up: token of each sorted row; down: nullptr
  const void* w0;            // dense weights [E, N, K] (down, or gate)
  const void* w1;            // dense up weights (gate|up only)
  const void* bias0;         // [E, N] or nullptr
  const void* bias1;
  const void* sh_w0;         // shared expert weights [N_sh, K_sh] or nullptr
  const void* sh_w1;
  int N, K;                  // routed experts
  int N_sh, K_sh;            // shared expert
  int E, E_all;
  const int32_t* offsets;
  const int32_t* tile_prefix;
  void* out;
  int ldo;
  int act;
  float alpha, limit;
};

template <typename TA, bool GATED>
__global__ __launch_bounds__(kThreads) void tiled_gemm_kernel(GemmArgs a) {
  __shared__ float As[BK][BM + 1];
  __shared__ float Bs0[BK][BN + 1];
  __shared__ float Bs1[GATED ? BK : 1][BN + 1];

  const int tile = blockIdx.x;
  const int total_tiles = a.tile_prefix[a.E_all];
  if (tile >= total_tiles) return;
  // expert of this tile: last e with tile_prefix[e] <= tile
  int lo = 0, hi = a.E_all - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (a.tile_prefix[mid] <= tile) lo = mid; else hi = mid - 1;
  }
  const int e = lo;
  const bool shared = e >= a.E;
  const int N = shared ? a.N_sh : a.N;
  const int K = shared ? a.K_sh : a.K;
  const int n0 = blockIdx.y * BN;
  if (n0 >= N) return;
  const int r0 = a.offsets[e] + (tile - a.tile_prefix[e]) * BM;
  const int r_end = a.offsets[e + 1];

  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const TA* A = static_cast<const TA*>(a.a);

  // shared-expert weights are a single [N_sh, K_sh] matrix: index it as expert 0
  const void* w0 = shared ? a.sh_w0 : a.w0;
  const void* w1 = shared ? a.sh_w1 : a.w1;
  const int we = shared ? 0 : e;

  float acc0[4][4] = {};
  float acc1[GATED ? 4 : 1][GATED ? 4 : 1] = {};

  // loader coordinates: 64 rows x 16 k, 4 consecutive k per thread
  const int lr = tid >> 2, lk = (tid & 3) * 4;
  const int ar = r0 + lr;
  long a_row = -1;
  if (ar < r_end) a_row = a.row_token ? a.row_token[ar] : ar;

  for (int k0 = 0; k0 < K; k0 += BK) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int kk = k0 + lk + q;
      As[lk + q][lr] = (a_row >= 0 && kk < K) ? load_f32(A, (size_t)a_row * a.lda + kk) : 0.f;
      const int n = n0 + lr;
      const bool ok = n < N && kk < K;
      if (shared) {
        Bs0[lk + q][lr] = ok ? load_f32(static_cast<const TA*>(w0), (size_t)n * K + kk) : 0.f;
        if constexpr (GATED) Bs1[lk + q][lr] = ok ? load_f32(static_cast<const TA*>(w1), (size_t)n * K + kk) : 0.f;
      } else {
        Bs0[lk + q][lr] = ok ? load_f32(static_cast<const TA*>(w0), ((size_t)we * N + n) * K + kk) : 0.f;
        if constexpr (GATED) Bs1[lk + q][lr] = ok ? load_f32(static_cast<const TA*>(w1), ((size_t)we * N + n) * K + kk) : 0.f;
      }
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      float av[4], b0[4], b1[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = As[kk][ty + 16 * i];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        b0[j] = Bs0[kk][tx + 16 * j];
        if constexpr (GATED) b1[j] = Bs1[kk][tx + 16 * j];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc0[i][j] = fmaf(av[i], b0[j], acc0[i][j]);
          if constexpr (GATED) acc1[i][j] = fmaf(av[i], b1[j], acc1[i][j]);
        }
    }
    __syncthreads();
  }

  TA* O = static_cast<TA*>(a.out);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = r0 + ty + 16 * i;
    if (r >= r_end) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx + 16 * j;
      if (n >= N) continue;
      float v0 = acc0[i][j];
      if (!shared && a.bias0) v0 += load_f32(static_cast<const TA*>(a.bias0), (size_t)e * N + n);
      if constexpr (GATED) {
        float v1 = acc1[i][j];
        if (!shared && a.bias1) v1 += load_f32(static_cast<const TA*>(a.bias1), (size_t)e * N + n);
        v0 = expert_act(shared ? 1 : a.act, v0, v1, a.alpha, a.limit);
      }
      store_f32(O, (size_t)r * a.ldo + n, v0);
    }
  }
}

template <typename TA, bool GATED>
hipError_t launch_t(const GemmArgs& a, int rows_all, int n_max, hipStream_t s) {
  dim3 grid((rows_all + BM - 1) / BM + a.E_all, (n_max + BN - 1) / BN);
  tiled_gemm_kernel<TA, GATED><<<grid, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

GemmArgs common_args(const Layer& L, const Work& W) {
  GemmArgs g{};
  g.E = L.E;
  g.E_all = L.n_experts_all();
  g.offsets = W.offsets;
  g.tile_prefix = W.tile_prefix;
  g.act = L.act;
  g.alpha = L.alpha;
  g.limit = L.limit;
  return g;
}

}  // namespace

hipError_t launch_gate_up(const Layer& L, const Work& W, hipStream_t s) {
  GemmArgs g = common_args(L, W);
  g.a = L.x; g.lda = L.d; g.row_token = W.row_token;
  g.w0 = L.wg; g.w1 = L.wu;
  g.bias0 = L.bg; g.bias1 = L.bu;
  g.sh_w0 = L.sh_wg; g.sh_w1 = L.sh_wu;
  g.N = L.F; g.K = L.d; g.N_sh = L.F_sh; g.K_sh = L.d;
  g.out = W.h; g.ldo = L.F_max();
  const int rows = L.rows_all(), nmax = L.F_max();
  if (L.dt != MOE_F32) return hipErrorInvalidValue;  // bf16 and MXFP4 layers take the MFMA kernels
  return launch_t<float, true>(g, rows, nmax, s);
}

hipError_t launch_down(const Layer& L, const Work& W, hipStream_t s) {
  GemmArgs g = common_args(L, W);
  g.a = W.h; g.lda = L.F_max(); g.row_token = nullptr;
  g.w0 = L.wd;
  g.bias0 = L.bd;
  g.sh_w0 = L.sh_wd;
  g.N = L.d; g.K = L.F; g.N_sh = L.d; g.K_sh = L.F_sh;
  g.out = W.y; g.ldo = L.d;
  const int rows = L.rows_all();
  if (L.dt != MOE_F32) return hipErrorInvalidValue;
  return launch_t<float, false>(g, rows, L.d, s);
}

}  // namespace moe
