// Host side of the C ABI declared in moe_ffn.h: argument checks, workspace
// layout, and the launch sequence route -> permute -> gate|up -> down ->
// combine on the caller's stream.  Nothing here allocates device memory or
// synchronises, except the opt-in stage timer (moe_ffn_profile_*).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "moe_internal.h"

namespace moe {
namespace {

thread_local char g_detail[512] = "";

moe_status fail(moe_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_detail, sizeof(g_detail), fmt, ap);
  va_end(ap);
  return st;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  auto pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
  return pa < pb + nb && pb < pa + na;
}

// ---- opt-in stage timer ----------------------------------------------------
struct Profiler {
  std::mutex mu;
  unsigned mask = 0;
  std::vector<hipEvent_t> begin, end;
  std::vector<int> stage_of;  // stage of each used pair
  size_t used = 0;
} g_prof;

constexpr size_t kProfPairs = 8192;

struct StageTimer {
  hipStream_t s;
  int stage;
  long slot = -1;
  StageTimer(hipStream_t s_, int stage_) : s(s_), stage(stage_) {
    if (!(g_prof.mask & (1u << stage))) return;
    std::lock_guard<std::mutex> lk(g_prof.mu);
    if (g_prof.used >= g_prof.begin.size()) return;
    slot = static_cast<long>(g_prof.used++);
    g_prof.stage_of[slot] = stage;
    hipEventRecord(g_prof.begin[slot], s);
  }
  ~StageTimer() {
    if (slot >= 0) hipEventRecord(g_prof.end[slot], s);
  }
};

// ---- checks ----------------------------------------------------------------
moe_status check_common(const Layer& L) {
  if (L.T < 0) return fail(MOE_ERR_INVALID_ARG, "T = %d < 0", L.T);
  if (L.d < 1 || L.F < 1) return fail(MOE_ERR_INVALID_ARG, "d = %d, d_ff = %d must be >= 1", L.d, L.F);
  if (L.E < 1) return fail(MOE_ERR_INVALID_ARG, "E = %d must be >= 1", L.E);
  if (L.k < 1 || L.k > L.E) return fail(MOE_ERR_INVALID_ARG, "k = %d must be in [1, E = %d]", L.k, L.E);
  if (L.E > 256) return fail(MOE_ERR_UNSUPPORTED, "E = %d > 256", L.E);
  if (L.k > 16) return fail(MOE_ERR_UNSUPPORTED, "k = %d > 16", L.k);
  if ((long long)L.T * L.k >= (1ll << 26)) return fail(MOE_ERR_UNSUPPORTED, "T * k = %lld >= 2^26", (long long)L.T * L.k);
  if (L.dt != MOE_F32 && L.dt != MOE_BF16) return fail(MOE_ERR_INVALID_ARG, "unknown dtype %d", L.dt);
  const int q = L.wfmt == WF_AFF8 ? 64 : lowbit_format(L.wfmt) ? 32 : 8;
  if (L.d % q || L.F % q) return fail(MOE_ERR_UNSUPPORTED, "d = %d and d_ff = %d must be multiples of %d", L.d, L.F, q);
  if (lowbit_format(L.wfmt)) {
    // the low-bit kernels address one expert's codes and the activation
    // rows with 32-bit offsets
    const unsigned long long code_bytes = (unsigned long long)L.d * L.F * code_bits(L.wfmt) / 8;
    if (code_bytes >= (1ull << 32))
      return fail(MOE_ERR_UNSUPPORTED, "d * d_ff = %lld: an expert's codes reach 2^32 bytes", (long long)L.d * L.F);
    if ((unsigned long long)L.rows_all() * (L.d > L.F ? L.d : L.F) >= (1ull << 32))
      return fail(MOE_ERR_UNSUPPORTED, "T * k * max(d, d_ff) >= 2^32 with low-bit weights");
  }
  if (L.mx_act) {
    // whole 64-k MFMA steps; 32-bit offsets of the MXFP8 activation rows
    if (L.d % 64 || L.F % 64)
      return fail(MOE_ERR_UNSUPPORTED, "d = %d and d_ff = %d must be multiples of 64 with MXFP8 activations", L.d, L.F);
    if ((unsigned long long)L.rows_all() * mx_row_bytes(L.d > L.F ? L.d : L.F) >= (1ull << 32))
      return fail(MOE_ERR_UNSUPPORTED, "T * k * max(d, d_ff) >= 2^32 with MXFP8 activations");
  }
  if (L.act != MOE_ACT_CLIPPED_SWIGLU && L.act != MOE_ACT_SILU) return fail(MOE_ERR_INVALID_ARG, "unknown activation %d", L.act);
  if (L.act == MOE_ACT_CLIPPED_SWIGLU) {
    if (!(L.limit > 0.f) || !std::isfinite(L.limit)) return fail(MOE_ERR_INVALID_ARG, "limit = %g must be finite and > 0", (double)L.limit);
    if (!std::isfinite(L.alpha)) return fail(MOE_ERR_INVALID_ARG, "alpha must be finite");
  }
  if (L.grouped) {
    if (L.n_group < 1 || L.E % L.n_group) return fail(MOE_ERR_INVALID_ARG, "n_group = %d must divide E = %d", L.n_group, L.E);
    if (L.n_group > 64) return fail(MOE_ERR_UNSUPPORTED, "n_group = %d > 64", L.n_group);
    if (L.topk_group < 1 || L.topk_group > L.n_group)
      return fail(MOE_ERR_INVALID_ARG, "topk_group = %d must be in [1, n_group = %d]", L.topk_group, L.n_group);
    if (L.k > L.topk_group * (L.E / L.n_group))
      return fail(MOE_ERR_INVALID_ARG, "k = %d exceeds the %d experts of topk_group groups", L.k, L.topk_group * (L.E / L.n_group));
    if (!std::isfinite(L.rsf)) return fail(MOE_ERR_INVALID_ARG, "routed_scaling_factor must be finite");
    if (L.score != MOE_SCORE_SOFTMAX && L.score != MOE_SCORE_SIGMOID) return fail(MOE_ERR_INVALID_ARG, "unknown score %d", L.score);
  }
  if (L.has_shared()) {
    if (!L.sh_wu || !L.sh_wd) return fail(MOE_ERR_INVALID_ARG, "shared_w_up and shared_w_down are required with shared_w_gate");
    if (L.F_sh < 1 || L.F_sh % 8) return fail(MOE_ERR_INVALID_ARG, "d_ff_shared = %d must be >= 1 and a multiple of 8", L.F_sh);
  }
  if (L.norm_w && (!(L.eps >= 0.f) || !std::isfinite(L.eps)))
    return fail(MOE_ERR_INVALID_ARG, "RMSNorm eps = %g must be finite and >= 0", (double)L.eps);
  if (L.T == 0) return MOE_OK;
  if (!L.x || !L.router_w || !L.out) return fail(MOE_ERR_INVALID_ARG, "x, router_w and out are required");
  if (lowbit_format(L.wfmt)) {
    if (!L.wg_codes || !L.wg_scales || !L.wu_codes || !L.wu_scales || !L.wd_codes || !L.wd_scales)
      return fail(MOE_ERR_INVALID_ARG, "all codes and scales are required");
    if (L.wfmt == WF_NVFP4 && !(std::isfinite(L.ts_g) && std::isfinite(L.ts_u) && std::isfinite(L.ts_d)))
      return fail(MOE_ERR_INVALID_ARG, "NVFP4 tensor scales must be finite");
    if ((L.wfmt == WF_AFF4 || L.wfmt == WF_AFF8) && (!L.wg_qbias || !L.wu_qbias || !L.wd_qbias))
      return fail(MOE_ERR_INVALID_ARG, "all affine biases are required");
  } else if (!L.wg || !L.wu || !L.wd) {
    return fail(MOE_ERR_INVALID_ARG, "w_gate, w_up and w_down are required");
  }
  // x, the router weight, the dense expert weights and the codes are read
  // with 16-byte vector loads and global -> LDS copies; every other array at
  // least element by element
  const auto off16 = [](const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 != 0; };
  if (off16(L.x) || off16(L.router_w)) return fail(MOE_ERR_INVALID_ARG, "x and router_w must be 16-byte aligned");
  if (lowbit_format(L.wfmt)) {
    if (off16(L.wg_codes) || off16(L.wu_codes) || off16(L.wd_codes))
      return fail(MOE_ERR_INVALID_ARG, "the code tensors must be 16-byte aligned");
  } else if (off16(L.wg) || off16(L.wu) || off16(L.wd)) {
    return fail(MOE_ERR_INVALID_ARG, "w_gate, w_up and w_down must be 16-byte aligned");
  }
  if (L.has_shared() && (off16(L.sh_wg) || off16(L.sh_wu) || off16(L.sh_wd)))
    return fail(MOE_ERR_INVALID_ARG, "the shared expert's weights must be 16-byte aligned");
  // the bf16 router (many tokens) reads the RMSNorm weight with 16-byte loads
  if (L.dt == MOE_BF16 && off16(L.norm_w)) return fail(MOE_ERR_INVALID_ARG, "the RMSNorm weight must be 16-byte aligned");
  {
    const size_t el = L.elt();
    const auto off = [](const void* p, size_t a) { return reinterpret_cast<uintptr_t>(p) % a != 0; };
    if (off(L.out, el) || off(L.router_b, el) || off(L.bg, el) || off(L.bu, el) || off(L.bd, el) ||
        off(L.norm_w, el) || off(L.x_resid, el) || off(L.e_bias, 4))
      return fail(MOE_ERR_INVALID_ARG, "out, the biases, the norm weight and the residual must be aligned to their element size");
    if ((L.wfmt == WF_AFF4 || L.wfmt == WF_AFF8) &&
        (off(L.wg_scales, 2) || off(L.wu_scales, 2) || off(L.wd_scales, 2) || off(L.wg_qbias, 2) ||
         off(L.wu_qbias, 2) || off(L.wd_qbias, 2)))
      return fail(MOE_ERR_INVALID_ARG, "the affine scales and biases (bf16) must be 2-byte aligned");
  }
  if (L.mx_act) {
    const uintptr_t sc = reinterpret_cast<uintptr_t>(L.wg_scales) | reinterpret_cast<uintptr_t>(L.wu_scales) |
                         reinterpret_cast<uintptr_t>(L.wd_scales);
    if (sc % 4) return fail(MOE_ERR_INVALID_ARG, "the scale tensors must be 4-byte aligned with MXFP8 activations");
  }
  const size_t xbytes = (size_t)L.T * L.d * L.elt();
  if (overlaps(L.out, xbytes, L.x, xbytes)) return fail(MOE_ERR_INVALID_ARG, "out overlaps x");
  return MOE_OK;
}

moe_status run(Layer& L, void* ws, size_t ws_bytes, hipStream_t s) {
  g_detail[0] = '\0';
  moe_status st = check_common(L);
  if (st != MOE_OK || L.T == 0) return st;
  Work W;
  const size_t need = carve_workspace(L, nullptr, &W);
  if (need == (size_t)-1) return fail(MOE_ERR_UNSUPPORTED, "workspace size overflows");
  if (!ws || ws_bytes < need) return fail(MOE_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws ? ws_bytes : (size_t)0);
  if (reinterpret_cast<uintptr_t>(ws) % kAlign) return fail(MOE_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (overlaps(L.out, (size_t)L.T * L.d * L.elt(), ws, need)) return fail(MOE_ERR_INVALID_ARG, "out overlaps the workspace");
  carve_workspace(L, ws, &W);

  // Expert stages: weight streaming with vector dot products for a few tokens
  // (every expert then holds at most kDecodeMaxTokens rows), grouped MFMA
  // GEMMs otherwise, vector-ALU tiles for fp32.
  enum { kDecode, kMfma, kLowbit, kMx, kTiled } path;
  if (L.dt == MOE_F32) path = kTiled;
  else if (L.mx_act) path = kMx;
  // MXFP4 weights (no shared expert) stream through the decode kernel for a few tokens
  else if (L.wfmt == WF_MXFP4 && L.T <= kDecodeMaxTokens && !L.has_shared()) path = kDecode;
  else if (lowbit_format(L.wfmt)) path = kLowbit;
  else if (L.T <= kDecodeMaxTokens) path = kDecode;
  else path = kMfma;
  // A shared expert (bf16) next to many-token routed experts: its gate|up
  // tiles run in the router's launch and its down tiles in the
  // permutation's (they need neither), so the routed launches are whole
  // waves of routed tiles.  A MoE block's router writes the normalised rows
  // the shared expert reads, so there the shared expert's tiles follow the
  // routed ones: in the same launches (bf16 experts) or in launches of the
  // dense bf16 GEMM restricted to the shared expert, queued after the routed
  // launch on the same stream (low-bit experts).
  const bool shared_beside = MOE_SHARED_BESIDE && (path == kMfma || path == kLowbit) && L.has_shared() && !L.norm_w &&
                             L.dt == MOE_BF16 && L.T > kDecodeMaxTokens && L.E <= kSharedBesideMaxE;
  const bool shared_apart = path == kLowbit && L.has_shared() && !shared_beside;
  const bool routed_only = shared_beside;

  hipError_t e;
  {
    StageTimer tm(s, MOE_STAGE_ROUTE);
    e = hipSuccess;
    // block prologue: the layer works on RMSNorm(x) from here on.  bf16 with
    // more than 16 tokens: the router normalises the rows it streams and
    // writes them to W.xn; otherwise a kernel of its own first.
    if (L.norm_w && (L.dt == MOE_F32 || L.T <= kDecodeMaxTokens)) {
      e = launch_rmsnorm(L, W, s);
      L.x = W.xn;
    }
    if (e == hipSuccess) e = shared_beside ? launch_route_shared_gate_up(L, W, s) : launch_route(L, W, s);
    if (L.norm_w) L.x = W.xn;
  }
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "route launch: %s", hipGetErrorString(e));
  {
    StageTimer tm(s, MOE_STAGE_PERMUTE);
    e = shared_beside ? launch_permute_shared_down(L, W, s) : launch_permute(L, W, s);
    // MXFP8 activations: x's conversion is independent of the routing; it is
    // timed with this stage so that the gate|up stage is the GEMM alone
    if (e == hipSuccess && L.mx_act) e = launch_mx_quant(L.x, L.d, L.T, L.d, W.xq, W.xs, mx_row_bytes(L.d), s);
  }
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "permute launch: %s", hipGetErrorString(e));
  {
    StageTimer tm(s, MOE_STAGE_GATE_UP);
    if (path == kMx) {
      e = launch_gate_up_mx(L, W, s);
    } else {
      e = path == kDecode ? launch_gate_up_decode(L, W, s)
          : path == kMfma ? launch_gate_up_mfma(L, W, s, routed_only)
          : path == kLowbit ? launch_gate_up_lowbit(L, W, s) : launch_gate_up(L, W, s);
    }
    if (e == hipSuccess && shared_apart) e = launch_gate_up_mfma_shared(L, W, s);
  }
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "gate|up launch: %s", hipGetErrorString(e));
  {
    StageTimer tm(s, MOE_STAGE_DOWN);
    if (path == kMx) {
      e = launch_mx_quant(W.h, L.F_max(), L.rows_all(), L.F, W.hq, W.hs, mx_row_bytes(L.F), s);
      if (e == hipSuccess) e = launch_down_mx(L, W, s);
    } else {
      e = path == kDecode ? launch_down_decode(L, W, s)
          : path == kMfma ? launch_down_mfma(L, W, s, routed_only)
          : path == kLowbit ? launch_down_lowbit(L, W, s) : launch_down(L, W, s);
    }
    if (e == hipSuccess && shared_apart) e = launch_down_mfma_shared(L, W, s);
  }
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "down launch: %s", hipGetErrorString(e));
  {
    StageTimer tm(s, MOE_STAGE_COMBINE);
    e = launch_combine(L, W, s);
  }
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "combine launch: %s", hipGetErrorString(e));
  return MOE_OK;
}

}  // namespace

moe_status run_layer(Layer& L, void* ws, size_t ws_bytes, hipStream_t s) { return run(L, ws, ws_bytes, s); }

moe_status set_error(moe_status st, const char* what) {
  snprintf(g_detail, sizeof(g_detail), "%s", what);
  return st;
}

void clear_error() { g_detail[0] = '\0'; }

size_t carve_workspace(const Layer& L, void* ws, Work* W) {
  const size_t P = (size_t)L.T * L.k;
  const size_t rows = (size_t)L.rows_all();
  const size_t nblk = ((size_t)L.T + kMinRouteTokens - 1) / kMinRouteTokens;
  const size_t Eall = (size_t)L.n_experts_all();
  size_t off = 0;
  char* base = static_cast<char*>(ws);
  auto take = [&](size_t bytes) -> void* {
    void* p = base ? base + off : nullptr;
    off += align_up(bytes);
    return p;
  };
  W->idx = static_cast<int32_t*>(take(P * 4));
  W->w = static_cast<float*>(take(P * 4));
  W->hist = static_cast<int32_t*>(take(nblk * L.E * 4));
  const bool split_route = L.dt != MOE_F32 && L.T <= kDecodeMaxTokens;
  W->route_part = static_cast<float*>(take(split_route ? (size_t)kRouteSplitK * 16 * L.E * 4 : 0));
  W->offsets = static_cast<int32_t*>(take((Eall + 1) * 4));
  W->tile_prefix = static_cast<int32_t*>(take((Eall + 1) * 4));
  W->tile_prefix_big = static_cast<int32_t*>(take((Eall + 1) * 4));
  W->tile_desc = static_cast<int32_t*>(take((size_t)max_big_tiles((int)rows, (int)Eall) * 16));
  W->sorted_pair = static_cast<int32_t*>(take(rows * 4));
  W->row_token = static_cast<int32_t*>(take(rows * 4));
  W->pos = static_cast<int32_t*>(take(P * 4));
  W->h = take(rows * (size_t)L.F_max() * L.elt());
  W->y = take(rows * (size_t)L.d * L.elt());
  W->xn = take(L.norm_w ? (size_t)L.T * L.d * L.elt() : 0);
  const size_t xrow = L.mx_act ? (size_t)mx_row_bytes(L.d) : 0, hrow = L.mx_act ? (size_t)mx_row_bytes(L.F) : 0;
  W->xq = static_cast<uint8_t*>(take((size_t)L.T * xrow));
  W->xs = static_cast<uint8_t*>(take((size_t)L.T * xrow / 32));
  W->hq = static_cast<uint8_t*>(take(rows * hrow));
  W->hs = static_cast<uint8_t*>(take(rows * hrow / 32));
  W->zrow = L.dt == MOE_BF16 ? take(zero_row_bytes(L)) : nullptr;
  return off;
}

}  // namespace moe

using moe::Layer;

namespace {
void apply_block(Layer& L, const moe_block* b) {
  if (!b) return;
  L.norm_w = b->norm_w;
  L.eps = b->eps;
  L.x_resid = b->residual ? L.x : nullptr;
}
}  // namespace

extern "C" {

size_t moe_ffn_workspace_bytes(int T, int d, int d_ff, int E, int k, moe_dtype dt, int grouped, int d_ff_shared) {
  return moe_block_workspace_bytes(nullptr, T, d, d_ff, E, k, dt, grouped, d_ff_shared);
}

size_t moe_block_workspace_bytes(const moe_block* block, int T, int d, int d_ff, int E, int k, moe_dtype dt,
                                 int grouped, int d_ff_shared) {
  if (T < 0 || d < 1 || d_ff < 1 || E < 1 || E > 256 || k < 1 || k > 16 || k > E || d_ff_shared < 0) return (size_t)-1;
  if ((long long)T * k >= (1ll << 26)) return (size_t)-1;
  if (!grouped && d_ff_shared > 0) return (size_t)-1;  // only group-routed layers have a shared expert
  if (T == 0) return 0;
  Layer L;
  L.T = T; L.d = d; L.F = d_ff; L.E = E; L.k = k; L.dt = dt;
  L.grouped = grouped ? 1 : 0;
  L.F_sh = d_ff_shared;
  static const char dummy = 0;
  if (d_ff_shared > 0) L.sh_wg = &dummy;
  if (block && block->norm_w) L.norm_w = &dummy;
  moe::Work W;
  return moe::carve_workspace(L, nullptr, &W);
}

moe_status moe_ffn_forward(const void* x, const void* router_w, const void* router_b,
                           const void* w_gate, const void* b_gate, const void* w_up, const void* b_up,
                           const void* w_down, const void* b_down, int T, int d, int d_ff, int E, int k,
                           float alpha, float limit, void* out, moe_dtype dt, void* workspace,
                           size_t workspace_bytes, moe_routing_out* routing, hipStream_t stream) {
  return moe_block_forward(nullptr, x, router_w, router_b, w_gate, b_gate, w_up, b_up, w_down, b_down, T, d,
                           d_ff, E, k, alpha, limit, out, dt, workspace, workspace_bytes, routing, stream);
}

moe_status moe_block_forward(const moe_block* block, const void* x, const void* router_w, const void* router_b,
                             const void* w_gate, const void* b_gate, const void* w_up, const void* b_up,
                             const void* w_down, const void* b_down, int T, int d, int d_ff, int E, int k,
                             float alpha, float limit, void* out, moe_dtype dt, void* workspace,
                             size_t workspace_bytes, moe_routing_out* routing, hipStream_t stream) {
  Layer L;
  L.x = x; L.router_w = router_w; L.router_b = router_b;
  L.wg = w_gate; L.bg = b_gate; L.wu = w_up; L.bu = b_up; L.wd = w_down; L.bd = b_down;
  L.T = T; L.d = d; L.F = d_ff; L.E = E; L.k = k;
  L.act = MOE_ACT_CLIPPED_SWIGLU; L.alpha = alpha; L.limit = limit;
  L.dt = dt; L.wfmt = dt == MOE_F32 ? moe::WF_F32 : moe::WF_BF16;
  L.out = out;
  if (routing) L.routing = *routing;
  apply_block(L, block);
  return moe::run(L, workspace, workspace_bytes, stream);
}

moe_status moe_ffn_forward_mxfp4(const void* x, const void* router_w, const void* router_b,
                                 const uint8_t* w_gate_codes, const uint8_t* w_gate_scales, const void* b_gate,
                                 const uint8_t* w_up_codes, const uint8_t* w_up_scales, const void* b_up,
                                 const uint8_t* w_down_codes, const uint8_t* w_down_scales, const void* b_down,
                                 int T, int d, int d_ff, int E, int k, float alpha, float limit, void* out,
                                 void* workspace, size_t workspace_bytes, moe_routing_out* routing,
                                 hipStream_t stream) {
  return moe_block_forward_mxfp4(nullptr, x, router_w, router_b, w_gate_codes, w_gate_scales, b_gate, w_up_codes,
                                 w_up_scales, b_up, w_down_codes, w_down_scales, b_down, T, d, d_ff, E, k, alpha,
                                 limit, out, workspace, workspace_bytes, routing, stream);
}

moe_status moe_block_forward_mxfp4(const moe_block* block, const void* x, const void* router_w,
                                   const void* router_b, const uint8_t* w_gate_codes, const uint8_t* w_gate_scales,
                                   const void* b_gate, const uint8_t* w_up_codes, const uint8_t* w_up_scales,
                                   const void* b_up, const uint8_t* w_down_codes, const uint8_t* w_down_scales,
                                   const void* b_down, int T, int d, int d_ff, int E, int k, float alpha,
                                   float limit, void* out, void* workspace, size_t workspace_bytes,
                                   moe_routing_out* routing, hipStream_t stream) {
  Layer L;
  L.x = x; L.router_w = router_w; L.router_b = router_b;
  L.wg_codes = w_gate_codes; L.wg_scales = w_gate_scales; L.bg = b_gate;
  L.wu_codes = w_up_codes; L.wu_scales = w_up_scales; L.bu = b_up;
  L.wd_codes = w_down_codes; L.wd_scales = w_down_scales; L.bd = b_down;
  L.T = T; L.d = d; L.F = d_ff; L.E = E; L.k = k;
  L.act = MOE_ACT_CLIPPED_SWIGLU; L.alpha = alpha; L.limit = limit;
  L.dt = MOE_BF16; L.wfmt = moe::WF_MXFP4;
  L.out = out;
  if (routing) L.routing = *routing;
  apply_block(L, block);
  return moe::run(L, workspace, workspace_bytes, stream);
}

size_t moe_ffn_workspace_bytes_mxfp8(int T, int d, int d_ff, int E, int k) {
  if (T < 0 || d < 1 || d_ff < 1 || E < 1 || E > 256 || k < 1 || k > 16 || k > E) return (size_t)-1;
  if ((long long)T * k >= (1ll << 26)) return (size_t)-1;
  if (T == 0) return 0;
  Layer L;
  L.T = T; L.d = d; L.F = d_ff; L.E = E; L.k = k; L.dt = MOE_BF16;
  L.wfmt = moe::WF_MXFP4; L.mx_act = 1;
  moe::Work W;
  return moe::carve_workspace(L, nullptr, &W);
}

moe_status moe_ffn_mxfp8_h_layout(int T, int d, int d_ff, int E, int k, size_t* codes_offset,
                                  size_t* scales_offset, int* row_bytes) {
  moe::g_detail[0] = '\0';
  if (moe_ffn_workspace_bytes_mxfp8(T, d, d_ff, E, k) == (size_t)-1)
    return moe::fail(MOE_ERR_INVALID_ARG, "sizes outside the limits");
  if (T == 0) return moe::fail(MOE_ERR_INVALID_ARG, "T = 0: the call has no workspace");
  Layer L;
  L.T = T; L.d = d; L.F = d_ff; L.E = E; L.k = k; L.dt = MOE_BF16;
  L.wfmt = moe::WF_MXFP4; L.mx_act = 1;
  moe::Work W;
  // carve at a nonzero base: the offsets are the pointers minus the base
  char* const base = reinterpret_cast<char*>(static_cast<uintptr_t>(1) << 20);
  moe::carve_workspace(L, base, &W);
  if (codes_offset) *codes_offset = static_cast<size_t>(reinterpret_cast<char*>(W.hq) - base);
  if (scales_offset) *scales_offset = static_cast<size_t>(reinterpret_cast<char*>(W.hs) - base);
  if (row_bytes) *row_bytes = moe::mx_row_bytes(d_ff);
  return MOE_OK;
}

moe_status moe_ffn_forward_mxfp4_mxfp8(const void* x, const void* router_w, const void* router_b,
                                       const uint8_t* w_gate_codes, const uint8_t* w_gate_scales, const void* b_gate,
                                       const uint8_t* w_up_codes, const uint8_t* w_up_scales, const void* b_up,
                                       const uint8_t* w_down_codes, const uint8_t* w_down_scales, const void* b_down,
                                       int T, int d, int d_ff, int E, int k, float alpha, float limit, void* out,
                                       void* workspace, size_t workspace_bytes, moe_routing_out* routing,
                                       hipStream_t stream) {
  Layer L;
  L.x = x; L.router_w = router_w; L.router_b = router_b;
  L.wg_codes = w_gate_codes; L.wg_scales = w_gate_scales; L.bg = b_gate;
  L.wu_codes = w_up_codes; L.wu_scales = w_up_scales; L.bu = b_up;
  L.wd_codes = w_down_codes; L.wd_scales = w_down_scales; L.bd = b_down;
  L.T = T; L.d = d; L.F = d_ff; L.E = E; L.k = k;
  L.act = MOE_ACT_CLIPPED_SWIGLU; L.alpha = alpha; L.limit = limit;
  L.dt = MOE_BF16; L.wfmt = moe::WF_MXFP4; L.mx_act = 1;
  L.out = out;
  if (routing) L.routing = *routing;
  return moe::run(L, workspace, workspace_bytes, stream);
}

moe_status moe_ffn_forward_mxfp8_mxfp8(const void* x, const void* router_w, const void* router_b,
                                       const uint8_t* w_gate_codes, const uint8_t* w_gate_scales, const void* b_gate,
                                       const uint8_t* w_up_codes, const uint8_t* w_up_scales, const void* b_up,
                                       const uint8_t* w_down_codes, const uint8_t* w_down_scales, const void* b_down,
                                       int T, int d, int d_ff, int E, int k, float alpha, float limit, void* out,
                                       void* workspace, size_t workspace_bytes, moe_routing_out* routing,
                                       hipStream_t stream) {
  Layer L;
  L.x = x; L.router_w = router_w; L.router_b = router_b;
  L.wg_codes = w_gate_codes; L.wg_scales = w_gate_scales; L.bg = b_gate;
  L.wu_codes = w_up_codes; L.wu_scales = w_up_scales; L.bu = b_up;
  L.wd_codes = w_down_codes; L.wd_scales = w_down_scales; L.bd = b_down;
  L.T = T; L.d = d; L.F = d_ff; L.E = E; L.k = k;
  L.act = MOE_ACT_CLIPPED_SWIGLU; L.alpha = alpha; L.limit = limit;
  L.dt = MOE_BF16; L.wfmt = moe::WF_MXFP8; L.mx_act = 1;
  L.out = out;
  if (routing) L.routing = *routing;
  return moe::run(L, workspace, workspace_bytes, stream);
}

moe_status moe_ffn_forward_nvfp4(const void* x, const void* router_w, const void* router_b,
                                 const uint8_t* w_gate_codes, const uint8_t* w_gate_scales, float w_gate_tensor_scale,
                                 const void* b_gate, const uint8_t* w_up_codes, const uint8_t* w_up_scales,
                                 float w_up_tensor_scale, const void* b_up, const uint8_t* w_down_codes,
                                 const uint8_t* w_down_scales, float w_down_tensor_scale, const void* b_down, int T,
                                 int d, int d_ff, int E, int k, float alpha, float limit, void* out, void* workspace,
                                 size_t workspace_bytes, moe_routing_out* routing, hipStream_t stream) {
  Layer L;
  L.x = x; L.router_w = router_w; L.router_b = router_b;
  L.wg_codes = w_gate_codes; L.wg_scales = w_gate_scales; L.bg = b_gate; L.ts_g = w_gate_tensor_scale;
  L.wu_codes = w_up_codes; L.wu_scales = w_up_scales; L.bu = b_up; L.ts_u = w_up_tensor_scale;
  L.wd_codes = w_down_codes; L.wd_scales = w_down_scales; L.bd = b_down; L.ts_d = w_down_tensor_scale;
  L.T = T; L.d = d; L.F = d_ff; L.E = E; L.k = k;
  L.act = MOE_ACT_CLIPPED_SWIGLU; L.alpha = alpha; L.limit = limit;
  L.dt = MOE_BF16; L.wfmt = moe::WF_NVFP4;
  L.out = out;
  if (routing) L.routing = *routing;
  return moe::run(L, workspace, workspace_bytes, stream);
}

moe_status moe_mxfp8_quantize(const void* x, int rows, int cols, uint8_t* codes, uint8_t* scales,
                              hipStream_t stream) {
  moe::g_detail[0] = '\0';
  if (rows < 0) return moe::fail(MOE_ERR_INVALID_ARG, "rows = %d < 0", rows);
  if (cols < 32 || cols % 32) return moe::fail(MOE_ERR_INVALID_ARG, "cols = %d must be a positive multiple of 32", cols);
  if (rows == 0) return MOE_OK;
  if ((long long)rows * cols >= (1ll << 40))
    return moe::fail(MOE_ERR_UNSUPPORTED, "rows * cols = %lld >= 2^40", (long long)rows * cols);
  if (!x || !codes || !scales) return moe::fail(MOE_ERR_INVALID_ARG, "x, codes and scales are required");
  if (reinterpret_cast<uintptr_t>(x) % 16 || reinterpret_cast<uintptr_t>(codes) % 16)
    return moe::fail(MOE_ERR_INVALID_ARG, "x and codes must be 16-byte aligned");
  const size_t n = (size_t)rows * cols;
  if (moe::overlaps(codes, n, x, 2 * n) || moe::overlaps(scales, n / 32, x, 2 * n) ||
      moe::overlaps(codes, n, scales, n / 32))
    return moe::fail(MOE_ERR_INVALID_ARG, "x, codes and scales must not overlap");
  const hipError_t e = moe::launch_mx_quant(x, cols, rows, cols, codes, scales, cols, stream);
  if (e != hipSuccess) return moe::fail(MOE_ERR_HIP, "quantize launch: %s", hipGetErrorString(e));
  return MOE_OK;
}

moe_status moe_ffn_forward_grouped(const void* x, const void* router_w, const void* router_b,
                                   const float* e_score_bias, const void* w_gate, const void* b_gate,
                                   const void* w_up, const void* b_up, const void* w_down, const void* b_down,
                                   const void* shared_w_gate, const void* shared_w_up, const void* shared_w_down,
                                   int d_ff_shared, int T, int d, int d_ff, int E, int k, int n_group,
                                   int topk_group, int norm_topk_prob, float routed_scaling_factor,
                                   moe_score score, moe_act act, float alpha, float limit, void* out,
                                   moe_dtype dt, void* workspace, size_t workspace_bytes,
                                   moe_routing_out* routing, hipStream_t stream) {
  return moe_block_forward_grouped(nullptr, x, router_w, router_b, e_score_bias, w_gate, b_gate, w_up, b_up,
                                   w_down, b_down, shared_w_gate, shared_w_up, shared_w_down, d_ff_shared, T, d,
                                   d_ff, E, k, n_group, topk_group, norm_topk_prob, routed_scaling_factor, score,
                                   act, alpha, limit, out, dt, workspace, workspace_bytes, routing, stream);
}

moe_status moe_block_forward_grouped(const moe_block* block, const void* x, const void* router_w,
                                     const void* router_b, const float* e_score_bias, const void* w_gate,
                                     const void* b_gate, const void* w_up, const void* b_up, const void* w_down,
                                     const void* b_down, const void* shared_w_gate, const void* shared_w_up,
                                     const void* shared_w_down, int d_ff_shared, int T, int d, int d_ff, int E,
                                     int k, int n_group, int topk_group, int norm_topk_prob,
                                     float routed_scaling_factor, moe_score score, moe_act act, float alpha,
                                     float limit, void* out, moe_dtype dt, void* workspace,
                                     size_t workspace_bytes, moe_routing_out* routing, hipStream_t stream) {
  Layer L;
  L.x = x; L.router_w = router_w; L.router_b = router_b; L.e_bias = e_score_bias;
  L.wg = w_gate; L.bg = b_gate; L.wu = w_up; L.bu = b_up; L.wd = w_down; L.bd = b_down;
  L.sh_wg = shared_w_gate; L.sh_wu = shared_w_up; L.sh_wd = shared_w_down;
  L.F_sh = shared_w_gate ? d_ff_shared : 0;
  L.T = T; L.d = d; L.F = d_ff; L.E = E; L.k = k;
  L.grouped = 1; L.n_group = n_group; L.topk_group = topk_group; L.norm = norm_topk_prob ? 1 : 0;
  L.rsf = routed_scaling_factor; L.score = score;
  L.act = act; L.alpha = alpha; L.limit = limit;
  L.dt = dt; L.wfmt = dt == MOE_F32 ? moe::WF_F32 : moe::WF_BF16;
  L.out = out;
  if (routing) L.routing = *routing;
  apply_block(L, block);
  return moe::run(L, workspace, workspace_bytes, stream);
}

moe_status moe_block_forward_grouped_affine(const moe_block* block, const moe_affine_experts* experts,
                                            const void* x, const void* router_w, const void* router_b,
                                            const float* e_score_bias, const void* b_gate, const void* b_up,
                                            const void* b_down, const void* shared_w_gate, const void* shared_w_up,
                                            const void* shared_w_down, int d_ff_shared, int T, int d, int d_ff,
                                            int E, int k, int n_group, int topk_group, int norm_topk_prob,
                                            float routed_scaling_factor, moe_score score, moe_act act, float alpha,
                                            float limit, void* out, void* workspace, size_t workspace_bytes,
                                            moe_routing_out* routing, hipStream_t stream) {
  moe::g_detail[0] = '\0';
  if (!experts) return moe::fail(MOE_ERR_INVALID_ARG, "experts is required");
  if (experts->bits != 4 && experts->bits != 8)
    return moe::fail(MOE_ERR_UNSUPPORTED, "affine experts with %d bits (4 or 8 supported)", experts->bits);
  Layer L;
  L.x = x; L.router_w = router_w; L.router_b = router_b; L.e_bias = e_score_bias;
  L.wg_codes = experts->gate_q; L.wg_scales = static_cast<const uint8_t*>(experts->gate_scales);
  L.wg_qbias = experts->gate_biases;
  L.wu_codes = experts->up_q; L.wu_scales = static_cast<const uint8_t*>(experts->up_scales);
  L.wu_qbias = experts->up_biases;
  L.wd_codes = experts->down_q; L.wd_scales = static_cast<const uint8_t*>(experts->down_scales);
  L.wd_qbias = experts->down_biases;
  L.bg = b_gate; L.bu = b_up; L.bd = b_down;
  L.sh_wg = shared_w_gate; L.sh_wu = shared_w_up; L.sh_wd = shared_w_down;
  L.F_sh = shared_w_gate ? d_ff_shared : 0;
  L.T = T; L.d = d; L.F = d_ff; L.E = E; L.k = k;
  L.grouped = 1; L.n_group = n_group; L.topk_group = topk_group; L.norm = norm_topk_prob ? 1 : 0;
  L.rsf = routed_scaling_factor; L.score = score;
  L.act = act; L.alpha = alpha; L.limit = limit;
  L.dt = MOE_BF16; L.wfmt = experts->bits == 4 ? moe::WF_AFF4 : moe::WF_AFF8;
  L.out = out;
  if (routing) L.routing = *routing;
  apply_block(L, block);
  return moe::run(L, workspace, workspace_bytes, stream);
}

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
  }
  return "MOE_UNKNOWN_STATUS";
}

const char* moe_last_error_detail(void) { return moe::g_detail; }

moe_status moe_ffn_profile_enable(unsigned stage_mask) {
  using moe::g_prof;
  std::lock_guard<std::mutex> lk(g_prof.mu);
  if (stage_mask && g_prof.begin.empty()) {
    g_prof.begin.resize(moe::kProfPairs);
    g_prof.end.resize(moe::kProfPairs);
    g_prof.stage_of.assign(moe::kProfPairs, -1);
    for (size_t i = 0; i < moe::kProfPairs; ++i) {
      if (hipEventCreate(&g_prof.begin[i]) != hipSuccess || hipEventCreate(&g_prof.end[i]) != hipSuccess)
        return moe::fail(MOE_ERR_HIP, "hipEventCreate failed");
    }
  }
  g_prof.mask = stage_mask;
  g_prof.used = 0;
  return MOE_OK;
}

moe_status moe_ffn_profile_read(double* ms, int* launches, int n_stages) {
  using moe::g_prof;
  std::lock_guard<std::mutex> lk(g_prof.mu);
  for (int i = 0; i < n_stages; ++i) {
    if (ms) ms[i] = 0.0;
    if (launches) launches[i] = 0;
  }
  for (size_t i = 0; i < g_prof.used; ++i) {
    const int st = g_prof.stage_of[i];
    if (hipEventSynchronize(g_prof.end[i]) != hipSuccess) return moe::fail(MOE_ERR_HIP, "hipEventSynchronize failed");
    float t = 0.f;
    if (hipEventElapsedTime(&t, g_prof.begin[i], g_prof.end[i]) != hipSuccess)
      return moe::fail(MOE_ERR_HIP, "hipEventElapsedTime failed");
    if (st >= 0 && st < n_stages) {
      if (ms) ms[st] += t;
      if (launches) launches[st] += 1;
    }
  }
  g_prof.used = 0;
  return MOE_OK;
}

}  // extern "C"
