// Internal declarations shared by the host dispatcher and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe_ffn.h"

namespace moe {

// Storage format of the expert weights.
// WF_AFF4 / WF_AFF8: affine group-quantized codes (4 bits, groups of 32 /
// 8 bits, groups of 64) with bf16 scales and biases.  WF_MXFP8: E4M3 codes
// with an e8m0 scale per 32 (only with MXFP8 activations, on the scaled MFMA).
// WF_NVFP4: e2m1 codes with an E4M3 scale per 16 and an fp32 tensor scale.
enum WeightFmt : int { WF_F32 = 0, WF_BF16 = 1, WF_MXFP4 = 2, WF_AFF4 = 3, WF_AFF8 = 4, WF_MXFP8 = 5, WF_NVFP4 = 6 };
inline bool lowbit_format(int wfmt) { return wfmt >= WF_MXFP4; }
inline int code_bits(int wfmt) { return wfmt == WF_AFF8 || wfmt == WF_MXFP8 ? 8 : 4; }

// Tokens handled by one block of the permute kernel.  Router blocks cover
// route_block_tokens() tokens, a divisor of this.
constexpr int kPermuteTokens = 64;
// Smallest router block (rows of the per-block expert count table).
constexpr int kMinRouteTokens = 16;
// Largest token count that takes the weight-streaming (decode) expert path:
// an expert then has at most this many rows, one MFMA column tile.
constexpr int kDecodeMaxTokens = 16;
// Few-token (T <= kDecodeMaxTokens, bf16) router: the input dimension is
// split over this many blocks per 16-expert group, whose partial logits a
// second kernel adds in a fixed order before choosing the experts.
constexpr int kRouteSplitK = 16;
// Rows per M-tile of the tiled grouped GEMMs (the permute kernel writes the
// per-expert tile prefix for this size).
constexpr int kTileM = 64;
// Rows per M-tile of the MFMA grouped GEMMs.
constexpr int kTileMBig = 256;
// Bytes of one MXFP8 activation row of K elements in the workspace: whole
// 128-element stages of the scaled-MFMA GEMMs, zero codes past K.
inline int mx_row_bytes(int K) { return (K + 127) / 128 * 128; }
// Upper bound on the number of 256-row tiles of a call.
inline int max_big_tiles(int rows_all, int E_all) { return (rows_all + kTileMBig - 1) / kTileMBig + E_all; }

// One call's arguments after validation.
struct Layer {
  const void* x = nullptr;
  const void* router_w = nullptr;
  const void* router_b = nullptr;
  const float* e_bias = nullptr;
  const void* wg = nullptr;
  const void* bg = nullptr;
  const void* wu = nullptr;
  const void* bu = nullptr;
  const void* wd = nullptr;
  const void* bd = nullptr;
  const uint8_t* wg_codes = nullptr;
  const uint8_t* wg_scales = nullptr;
  const uint8_t* wu_codes = nullptr;
  const uint8_t* wu_scales = nullptr;
  const uint8_t* wd_codes = nullptr;
  const uint8_t* wd_scales = nullptr;     // MXFP4: e8m0 bytes; affine: bf16 scales
  const void* wg_qbias = nullptr;         // affine: bf16 biases of the codes
  const void* wu_qbias = nullptr;
  const void* wd_qbias = nullptr;
  float ts_g = 1.f, ts_u = 1.f, ts_d = 1.f;  // NVFP4 tensor scales
  const void* sh_wg = nullptr;
  const void* sh_wu = nullptr;
  const void* sh_wd = nullptr;
  int F_sh = 0;
  int T = 0, d = 0, F = 0, E = 0, k = 0;
  int grouped = 0, n_group = 1, topk_group = 1, norm = 0;
  float rsf = 1.f;
  int score = MOE_SCORE_SOFTMAX;
  int act = MOE_ACT_CLIPPED_SWIGLU;
  float alpha = 1.702f, limit = 7.f;
  int dt = MOE_BF16;
  int wfmt = WF_BF16;
  void* out = nullptr;
  moe_routing_out routing{nullptr, nullptr, nullptr, nullptr};
  // MoE block: RMSNorm scale (nullptr: none) and epsilon; x_resid: the rows
  // added to the output (nullptr: no residual).  After the norm, x points at
  // the normalised rows and x_resid still at the caller's x.
  const void* norm_w = nullptr;
  float eps = 0.f;
  const void* x_resid = nullptr;
  // MXFP4 experts on the scaled MFMA: the expert GEMMs' activation operands
  // (x rows, h) are converted to MXFP8 first
  int mx_act = 0;

  bool has_shared() const { return sh_wg != nullptr; }
  int n_experts_all() const { return E + (has_shared() ? 1 : 0); }
  int pairs() const { return T * k; }
  int rows_all() const { return T * k + (has_shared() ? T : 0); }
  int F_max() const { return F_sh > F ? F_sh : F; }
  size_t elt() const { return dt == MOE_F32 ? 4 : 2; }
};

// Device buffers carved out of the caller's workspace.
struct Work {
  int32_t* idx = nullptr;          // [T*k] chosen experts
  float* w = nullptr;              // [T*k] routing weights
  int32_t* hist = nullptr;         // [n_route_blocks * E] per-block expert counts
  float* route_part = nullptr;     // few-token router: [kRouteSplitK][16][E] partial logits
  int32_t* offsets = nullptr;      // [E_all + 1] row offsets of each expert (shared last)
  int32_t* tile_prefix = nullptr;  // [E_all + 1] first 64-row M-tile of each expert
  int32_t* tile_prefix_big = nullptr;  // [E_all + 1] first 256-row M-tile of each expert
  int32_t* tile_desc = nullptr;    // [max 256-row tiles][4]: expert, first row, end row, 0
  int32_t* sorted_pair = nullptr;  // [rows_all] pair id of each sorted row (shared rows: -1)
  int32_t* row_token = nullptr;    // [rows_all] token of each sorted row
  int32_t* pos = nullptr;          // [T*k] sorted row of each pair
  void* h = nullptr;               // [rows_all, F_max] hidden activation (dt)
  void* y = nullptr;               // [rows_all, d] expert outputs (dt)
  void* xn = nullptr;              // block with a norm: [T, d] normalised rows (dt)
  uint8_t* xq = nullptr;           // MXFP8 activations: x as E4M3 codes [T, mx_row_bytes(d)]
  uint8_t* xs = nullptr;           //   and e8m0 scales [T, mx_row_bytes(d) / 32]
  uint8_t* hq = nullptr;           //   h as codes [rows, mx_row_bytes(d_ff)]
  uint8_t* hs = nullptr;           //   and scales [rows, mx_row_bytes(d_ff) / 32]
  void* zrow = nullptr;            // bf16: zero_row_bytes() of zeros, written by the permutation
};

// Bytes of the zero row: at least a bf16 row of max(d, F_max) elements and an
// MXFP8 code row (mx_row_bytes) of either.
inline size_t zero_row_bytes(const Layer& L) {
  const int m = L.d > L.F_max() ? L.d : L.F_max();
  return 2 * (size_t)m + 256;
}

// Byte size of the workspace and the layout of its buffers (ws == nullptr:
// size only).  Returns (size_t)-1 for sizes it cannot represent.
size_t carve_workspace(const Layer& L, void* ws, Work* W);

int route_block_tokens(const Layer& L);

// Checks L, then enqueues the whole layer on `s` with workspace ws (the body
// of every forward entry point).
moe_status run_layer(Layer& L, void* ws, size_t ws_bytes, hipStream_t s);
// Sets / clears the calling thread's error detail (moe_last_error_detail).
moe_status set_error(moe_status st, const char* what);
void clear_error();

// Kernel launchers (each enqueues one kernel on `s`).
hipError_t launch_route(const Layer& L, const Work& W, hipStream_t s);
hipError_t launch_permute(const Layer& L, const Work& W, hipStream_t s);
hipError_t launch_gate_up(const Layer& L, const Work& W, hipStream_t s);
hipError_t launch_down(const Layer& L, const Work& W, hipStream_t s);
hipError_t launch_gate_up_decode(const Layer& L, const Work& W, hipStream_t s);
hipError_t launch_down_decode(const Layer& L, const Work& W, hipStream_t s);
// routed_only: the tiles of experts [0, E), leaving a shared expert's to the
// _shared launchers; otherwise every expert's
hipError_t launch_gate_up_mfma(const Layer& L, const Work& W, hipStream_t s, bool routed_only);
hipError_t launch_down_mfma(const Layer& L, const Work& W, hipStream_t s, bool routed_only);
// low-bit expert weights (MXFP4, affine); the shared expert's tiles are skipped
hipError_t launch_gate_up_lowbit(const Layer& L, const Work& W, hipStream_t s);
hipError_t launch_down_lowbit(const Layer& L, const Work& W, hipStream_t s);
// the dense bf16 GEMMs restricted to the shared expert's tiles
hipError_t launch_gate_up_mfma_shared(const Layer& L, const Work& W, hipStream_t s);
hipError_t launch_down_mfma_shared(const Layer& L, const Work& W, hipStream_t s);
// bf16 layers with a shared expert, more than kDecodeMaxTokens tokens, at most
// kSharedBesideMaxE routed experts and no RMSNorm prologue: the router's
// launch also runs the shared expert's gate|up tiles, the permutation's
// launch its down tiles.  (The router block's LDS for more experts does not
// fit beside the GEMM tile's.)
constexpr int kSharedBesideMaxE = 128;
// 0: the shared expert's tiles always follow the routed ones (kept for
// timing the two schedules against each other).
#ifndef MOE_SHARED_BESIDE
#define MOE_SHARED_BESIDE 1
#endif
hipError_t launch_route_shared_gate_up(const Layer& L, const Work& W, hipStream_t s);
hipError_t launch_permute_shared_down(const Layer& L, const Work& W, hipStream_t s);
// MXFP8 activations times MXFP4 weights on the scaled MFMA
hipError_t launch_gate_up_mx(const Layer& L, const Work& W, hipStream_t s);
hipError_t launch_down_mx(const Layer& L, const Work& W, hipStream_t s);
// MXFP8 conversion of R bf16 rows of K elements (row stride lds elements)
// into codes [R, ldq] and scales [R, ldq / 32]; blocks past K get zero codes
// and scale byte 0.  K % 32 == 0, ldq % 32 == 0, ldq >= K.
hipError_t launch_mx_quant(const void* src, int lds, int R, int K, uint8_t* q, uint8_t* sc, int ldq, hipStream_t s);
hipError_t launch_combine(const Layer& L, const Work& W, hipStream_t s);
hipError_t launch_rmsnorm(const Layer& L, const Work& W, hipStream_t s);

}  // namespace moe
