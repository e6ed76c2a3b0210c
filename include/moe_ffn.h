/*
 * moe_ffn.h -- C ABI of an MI355X (gfx950) Mixture-of-Experts feed-forward layer.
 *
 * One call runs one MoE-FFN layer forward for T tokens on the caller's HIP
 * stream:
 *
 *   1. router logits   l[t,e] = x[t,:] . router_w[e,:] + router_b[e]     (fp32)
 *   2. routing         top-k experts per token and their weights
 *   3. permutation     (token, slot) pairs sorted by expert, stably
 *   4. gate|up         g = x W_gate[e]^T + b_gate[e], u = x W_up[e]^T + b_up[e],
 *                      h = act(g, u)
 *   5. down            y = h W_down[e]^T + b_down[e]
 *   6. combine         out[t] = sum_j w[t,j] * y[t,j]  (+ shared expert(x_t))
 *
 * Sources (web pages on the MoE layers of GPT-OSS and GLM4-MoE-Lite):
 *   - "Implementation:Ollama Ollama Imagegen GPT OSS", Description / Signature:
 *     clipped SwiGLU (gate clipped to [0, limit], up to [-limit, limit], fixed
 *     sigmoid scaling alpha = 1.702), num_local_experts, num_experts_per_tok,
 *     swiglu_limit.
 *   - MaxText GPT-OSS weight mapping, "MoE Router" and "MOE EXPERTS" blocks:
 *     router kernel + bias; separate gate_proj / up_proj kernels and biases;
 *     down projection (mlp2) weight and bias.
 *   - glm4_moe_lite.go: MoEGate.Forward (sigmoid scores, correction bias used
 *     for selection only, top-k, renormalisation when k > 1 and
 *     norm_topk_prob, routed_scaling_factor), SwitchMLP.Forward (stacked
 *     [E, out, in] expert weights, sort of the flattened expert indices and
 *     its inverse), SharedExperts.Forward and MoE.Forward (weighted sum, then
 *     shared experts added), Config (n_group, topk_group).
 *   - "GPT-OSS 20B GGUF with MoE CPU Offloading Support", Model
 *     Specifications: MXFP4 expert weights.  The MXFP4 bit layout is the OCP
 *     Microscaling (MX) v1.0 one (e2m1 elements, one e8m0 scale per 32).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers.  Every array pointer is a DEVICE pointer owned by the caller.
 *   The library never allocates, frees or synchronises device memory, keeps
 *   no state between calls (except the opt-in profiler below) and is
 *   reentrant.  Concurrent calls need distinct workspaces.  `out` must not
 *   overlap any input or the workspace.
 * Layouts.  Row-major and contiguous:
 *   x [T, d]; router_w [E, d]; router_b [E];
 *   w_gate, w_up [E, d_ff, d]; b_gate, b_up [E, d_ff];
 *   w_down [E, d, d_ff]; b_down [E, d]; out [T, d].
 *   Weights use the [out, in] convention: the reduction dimension is the
 *   contiguous one.
 * Element type.  `dt` gives the type of x, the router weight and bias, the
 *   dense expert weights, all expert biases and out (MOE_F32 or MOE_BF16).
 *   Router logits, routing weights, accumulation and the activation are fp32;
 *   with MOE_BF16 the hidden activation h and the expert outputs y are stored
 *   as bf16 between kernels.
 * Routing outputs.  `routing` may be NULL; each of its fields may be NULL.
 *   Non-NULL fields are filled (device pointers, caller-owned).
 * Workspace.  `workspace` is device memory of at least
 *   moe_ffn_workspace_bytes(...) bytes, 256-byte aligned; its contents on
 *   entry do not matter and are clobbered.  Every call's kernels read and
 *   write it, so two calls may share a workspace only when one is ordered
 *   after the other (the same stream, or an event between their streams).
 * Stream.  All work is enqueued on `stream` (0 = the null stream), in launch
 *   order; the library creates no stream or event of its own outside the
 *   opt-in stage timer.  The call returns without waiting for the GPU.
 * Errors.  Every argument is checked on the host before anything is
 *   enqueued.  On an error nothing is launched, `out` and the workspace are
 *   untouched and a non-zero status is returned; moe_last_error_detail()
 *   then describes it.  T == 0 is a valid no-op.  A launch failure returns
 *   MOE_ERR_HIP.  Faults inside kernels surface at the caller's next
 *   synchronisation.
 * Limits.  1 <= E <= 256, 1 <= k <= min(E, 16), d and d_ff multiples of 8
 *   (of 32 for MXFP4 weights), T * k < 2^26.
 * Alignment.  x, router_w, the dense expert weights (routed and shared),
 *   the code tensors and, for bf16 blocks, the RMSNorm weight are read with
 *   16-byte vector loads and must be 16-byte aligned; out, the biases, the
 *   residual, the fp32 norm weight and the affine scale and bias tables must
 *   be aligned to their element size.  Otherwise
 *   MOE_ERR_INVALID_ARG.  (Whole allocations from hipMalloc or torch are.)
 */
#ifndef MOE_FFN_H
#define MOE_FFN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,  /* NULL required pointer, out-of-range size or parameter */
  MOE_ERR_UNSUPPORTED = 2,  /* valid layer outside the limits listed above */
  MOE_ERR_WORKSPACE = 3,    /* workspace missing, too small or misaligned */
  MOE_ERR_HIP = 4           /* a HIP launch or runtime call failed */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Activation of the expert MLP.
 *   MOE_ACT_CLIPPED_SWIGLU: g' = min(max(g, 0), limit), u' = min(max(u, -limit), limit),
 *                           h = g' * sigmoid(alpha * g') * u'   (GPT-OSS page, Description)
 *   MOE_ACT_SILU:           h = g * sigmoid(g) * u             (glm4_moe_lite.go, SwitchMLP) */
typedef enum { MOE_ACT_CLIPPED_SWIGLU = 0, MOE_ACT_SILU = 1 } moe_act;

/* Expert score of grouped routing: softmax over all E logits, or the
 * element-wise sigmoid that glm4_moe_lite.go's MoEGate.Forward applies. */
typedef enum { MOE_SCORE_SOFTMAX = 0, MOE_SCORE_SIGMOID = 1 } moe_score;

typedef struct {
  int32_t* topk_idx;       /* [T, k]: chosen experts, best first (ties: lower index first) */
  float* topk_w;           /* [T, k]: routing weight of each chosen expert */
  int32_t* expert_offsets; /* [E + 1]: exclusive prefix sum of pairs per routed expert */
  int32_t* sorted_pair;    /* [T * k]: pair ids p = t*k + j sorted by (expert, p) */
} moe_routing_out;

/* Bytes of workspace a call with these sizes needs (pure host function).
 * grouped: nonzero for the group-routed layer (moe_ffn_forward_grouped and
 * its block and affine forms), zero for the GPT-OSS-style layers; only a
 * group-routed layer has a shared expert.  d_ff_shared = 0 when there is no
 * shared expert.  Returns 0 for T == 0 and (size_t)-1 for sizes outside the
 * limits or a shared expert with grouped == 0. */
size_t moe_ffn_workspace_bytes(int T, int d, int d_ff, int E, int k, moe_dtype dt, int grouped, int d_ff_shared);

/* GPT-OSS-style layer.
 * Routing: the k largest router logits per token (ties to the lower expert
 * index), weights = softmax over the k selected logits.  Activation: clipped
 * SwiGLU with `alpha` and `limit` (limit > 0).  router_b, b_gate, b_up,
 * b_down may be NULL (no bias); x, router_w, w_gate, w_up, w_down and out are
 * required when T > 0. */
moe_status moe_ffn_forward(const void* x, const void* router_w, const void* router_b,
                           const void* w_gate, const void* b_gate,
                           const void* w_up, const void* b_up,
                           const void* w_down, const void* b_down,
                           int T, int d, int d_ff, int E, int k, float alpha, float limit,
                           void* out, moe_dtype dt, void* workspace, size_t workspace_bytes,
                           moe_routing_out* routing, hipStream_t stream);

/* GPT-OSS-style layer with MXFP4 expert weights ("F16 base + MXFP4 expert
 * weights", GGUF page, Model Specifications).  Same as moe_ffn_forward with
 * dt = MOE_BF16, except that each expert weight is a pair:
 *   *_codes  uint8 [E, rows, cols/2]: e2m1 codes (bit 3 = sign), element 2i of
 *            a row in the low nibble, element 2i+1 in the high nibble;
 *   *_scales uint8 [E, rows, cols/32]: e8m0 scale 2^(byte-127) of each block of
 *            32 consecutive elements along cols (the input dimension).
 * (rows, cols) = (d_ff, d) for gate and up, (d, d_ff) for down.  x, router
 * weight and bias, expert biases and out are bf16.  d and d_ff must be
 * multiples of 32, d * d_ff < 2^33 and T * k * max(d, d_ff) < 2^32
 * (MOE_ERR_UNSUPPORTED otherwise).  A scale byte of 255 (NaN) yields NaN
 * outputs. */
moe_status moe_ffn_forward_mxfp4(const void* x, const void* router_w, const void* router_b,
                                 const uint8_t* w_gate_codes, const uint8_t* w_gate_scales, const void* b_gate,
                                 const uint8_t* w_up_codes, const uint8_t* w_up_scales, const void* b_up,
                                 const uint8_t* w_down_codes, const uint8_t* w_down_scales, const void* b_down,
                                 int T, int d, int d_ff, int E, int k, float alpha, float limit,
                                 void* out, void* workspace, size_t workspace_bytes,
                                 moe_routing_out* routing, hipStream_t stream);

/* GPT-OSS-style layer with NVFP4 expert weights (glm4_moe_lite.go
 * quantizationParams: NVFP4 = groups of 16, 4 bits; the layout is the
 * published NVFP4 one).  Same as moe_ffn_forward_mxfp4 except the scales:
 *   *_codes  uint8 [E, rows, cols/2]: e2m1 codes as for MXFP4;
 *   *_scales uint8 [E, rows, cols/16]: E4M3 codes (bit 7 sign, bits 6..3
 *            exponent with bias 7, bits 2..0 mantissa; S.1111.111 is NaN),
 *            one per 16 consecutive elements along cols;
 *   *_tensor_scale: fp32 factor of the whole tensor (finite, else
 *            MOE_ERR_INVALID_ARG).
 * W = e2m1(code) * e4m3(scale) * tensor_scale; the weights are rounded to
 * bf16 for the MFMA (exact when the product has at most 8 significant bits).
 * A NaN scale yields NaN outputs where its block is used.  Workspace as
 * moe_ffn_workspace_bytes(..., MOE_BF16, 0). */
moe_status moe_ffn_forward_nvfp4(const void* x, const void* router_w, const void* router_b,
                                 const uint8_t* w_gate_codes, const uint8_t* w_gate_scales, float w_gate_tensor_scale,
                                 const void* b_gate, const uint8_t* w_up_codes, const uint8_t* w_up_scales,
                                 float w_up_tensor_scale, const void* b_up, const uint8_t* w_down_codes,
                                 const uint8_t* w_down_scales, float w_down_tensor_scale, const void* b_down, int T,
                                 int d, int d_ff, int E, int k, float alpha, float limit, void* out, void* workspace,
                                 size_t workspace_bytes, moe_routing_out* routing, hipStream_t stream);

/* GPT-OSS-style MXFP4 layer on the gfx950 scaled MFMA (MXFP8 activations).
 * Arguments, layouts and routing as moe_ffn_forward_mxfp4; the expert GEMMs
 * differ: the rows entering gate|up (x) and down (h, after bias and
 * activation, rounded to bf16) are first converted to MXFP8 as
 * moe_mxfp8_quantize does (OCP Microscaling Formats v1.0 block conversion;
 * MXFP8 = 32-element groups of 8 bits in glm4_moe_lite.go
 * quantizationParams), and v_mfma_scale_f32_32x32x64_f8f6f4 multiplies the
 * E4M3 activation codes by the e2m1 weight codes with both block scales,
 * accumulating in fp32.  The result therefore differs from
 * moe_ffn_forward_mxfp4 by the activation rounding (E4M3 keeps 3 mantissa
 * bits).  The workspace is moe_ffn_workspace_bytes_mxfp8() bytes.
 * Requirements beyond moe_ffn_forward_mxfp4 (MOE_ERR_UNSUPPORTED /
 * MOE_ERR_INVALID_ARG otherwise): d and d_ff multiples of 64,
 * T * k * max(d, d_ff) rounded up to 128 below 2^32, x 16-byte aligned, the
 * three scale tensors 4-byte aligned. */
moe_status moe_ffn_forward_mxfp4_mxfp8(const void* x, const void* router_w, const void* router_b,
                                       const uint8_t* w_gate_codes, const uint8_t* w_gate_scales, const void* b_gate,
                                       const uint8_t* w_up_codes, const uint8_t* w_up_scales, const void* b_up,
                                       const uint8_t* w_down_codes, const uint8_t* w_down_scales, const void* b_down,
                                       int T, int d, int d_ff, int E, int k, float alpha, float limit, void* out,
                                       void* workspace, size_t workspace_bytes, moe_routing_out* routing,
                                       hipStream_t stream);

/* The same layer with MXFP8 expert weights (the MXFP8 mode of glm4_moe_lite.go
 * quantizationParams: groups of 32, 8 bits; OCP Microscaling Formats v1.0):
 *   *_codes  uint8 [E, rows, cols]: E4M3 codes (bit 7 sign, bits 6..3 exponent
 *            with bias 7, bits 2..0 mantissa; S.1111.111 is NaN);
 *   *_scales uint8 [E, rows, cols/32]: e8m0 scales as for MXFP4.
 * Everything else as moe_ffn_forward_mxfp4_mxfp8 (MXFP8 activations, the
 * scaled MFMA with E4M3 operands on both sides, the same workspace size and
 * requirements; one expert's codes below 2^32 bytes). */
moe_status moe_ffn_forward_mxfp8_mxfp8(const void* x, const void* router_w, const void* router_b,
                                       const uint8_t* w_gate_codes, const uint8_t* w_gate_scales, const void* b_gate,
                                       const uint8_t* w_up_codes, const uint8_t* w_up_scales, const void* b_up,
                                       const uint8_t* w_down_codes, const uint8_t* w_down_scales, const void* b_down,
                                       int T, int d, int d_ff, int E, int k, float alpha, float limit, void* out,
                                       void* workspace, size_t workspace_bytes, moe_routing_out* routing,
                                       hipStream_t stream);

/* Workspace bytes of moe_ffn_forward_mxfp4_mxfp8 and moe_ffn_forward_mxfp8_mxfp8 ((size_t)-1 for invalid
 * sizes, 0 for T == 0).  It adds the MXFP8 copies of x and h to the MXFP4
 * layer's workspace. */
size_t moe_ffn_workspace_bytes_mxfp8(int T, int d, int d_ff, int E, int k);

/* Where a call of moe_ffn_forward_mxfp4_mxfp8 or moe_ffn_forward_mxfp8_mxfp8
 * with these sizes leaves the MXFP8 form of the hidden activation h in its
 * workspace (pure host function).  After the call has run, and until the
 * workspace is used again, the workspace holds
 *   at byte *codes_offset:  uint8 [T * k, *row_bytes]: the E4M3 codes of h,
 *                           one row per (token, slot) pair in expert-sorted
 *                           order (row r belongs to pair sorted_pair[r] of
 *                           moe_routing_out), elements d_ff.. zero codes;
 *   at byte *scales_offset: uint8 [T * k, *row_bytes / 32]: their e8m0 scales.
 * The down GEMM consumes exactly these codes.  They are what a checker needs
 * to verify each rounding decision of h (E4M3 keeps 3 mantissa bits, so a
 * value within fp32 accumulation error of a rounding boundary has two
 * correct codes).  Output pointers may be NULL.  Errors: MOE_ERR_INVALID_ARG
 * for sizes outside the limits or T == 0. */
moe_status moe_ffn_mxfp8_h_layout(int T, int d, int d_ff, int E, int k, size_t* codes_offset,
                                  size_t* scales_offset, int* row_bytes);

/* MXFP8 conversion of bf16 rows, the activation step of
 * moe_ffn_forward_mxfp4_mxfp8 (OCP Microscaling Formats v1.0: E4M3 elements,
 * one e8m0 scale per 32 consecutive elements of a row).
 *   x      bf16 [rows, cols], device, 16-byte aligned; cols a positive multiple of 32.
 *   codes  uint8 [rows, cols], device, 16-byte aligned: E4M3 codes.
 *   scales uint8 [rows, cols/32], device: scale bytes.
 * Per block of 32 values: s = floor(log2(max |v|)) - 8 clamped to
 * [-127, 127], scale byte = s + 127, code = v / 2^s rounded to the nearest
 * E4M3 value, ties to even, magnitudes from 448 up giving 448 (the sign bit
 * is v's).  An all-zero block gets scale byte 0; a block holding a NaN or an
 * infinity gets scale byte 255 (NaN) and zero codes.  Enqueued on `stream`;
 * rows == 0 is a no-op.  The three buffers must not overlap.  Errors:
 * MOE_ERR_INVALID_ARG, or MOE_ERR_UNSUPPORTED for rows * cols >= 2^40
 * (nothing is launched). */
moe_status moe_mxfp8_quantize(const void* x, int rows, int cols, uint8_t* codes, uint8_t* scales,
                              hipStream_t stream);

/* GLM4-MoE-style layer with group-limited routing and optional shared expert
 * (glm4_moe_lite.go: Config, MoEGate.Forward, SharedExperts.Forward, MoE.Forward).
 * Routing per token:
 *   s  = softmax(l) over all E (score = MOE_SCORE_SOFTMAX) or sigmoid(l);
 *   s' = s + e_score_bias (fp32 [E], NULL = none; used for selection only);
 *   the E experts form n_group contiguous groups of E/n_group; a group's
 *   score is the largest s' in it; the topk_group best groups are kept (ties
 *   to the lower group index); the k best experts by s' among the kept
 *   groups are chosen (ties to the lower index);
 *   w = s[chosen]; if k > 1 and norm_topk_prob, w /= sum(w); w *= routed_scaling_factor.
 * Requirements: E % n_group == 0, 1 <= n_group <= 64, 1 <= topk_group <= n_group,
 * k <= topk_group * E / n_group.
 * Experts use `act` (with alpha/limit for MOE_ACT_CLIPPED_SWIGLU).  Biases may be NULL.
 * Shared expert: when shared_w_gate != NULL, shared_w_gate/shared_w_up
 * [d_ff_shared, d] and shared_w_down [d, d_ff_shared] (same dt, no bias)
 * form a SiLU-gated MLP applied to every token with weight 1 and added after
 * the routed sum; d_ff_shared must then be >= 1 and a multiple of 8. */
moe_status moe_ffn_forward_grouped(const void* x, const void* router_w, const void* router_b,
                                   const float* e_score_bias,
                                   const void* w_gate, const void* b_gate,
                                   const void* w_up, const void* b_up,
                                   const void* w_down, const void* b_down,
                                   const void* shared_w_gate, const void* shared_w_up,
                                   const void* shared_w_down, int d_ff_shared,
                                   int T, int d, int d_ff, int E, int k,
                                   int n_group, int topk_group, int norm_topk_prob,
                                   float routed_scaling_factor, moe_score score,
                                   moe_act act, float alpha, float limit,
                                   void* out, moe_dtype dt, void* workspace, size_t workspace_bytes,
                                   moe_routing_out* routing, hipStream_t stream);

/* ---- MoE block: RMSNorm in front of the layer, residual after it --------
 * glm4_moe_lite.go, MoEBlock.Forward (the half after attention): the MoE
 * input is PostAttentionLayerNorm(h), an RMSNorm with Config.RMSNormEps, and
 * the block returns h + MoE(...).  With a moe_block the layer computes
 *
 *   xn  = x / sqrt(mean(x^2) + eps) * norm_w     (norm_w != NULL; per token,
 *         over the d channels, fp32, rounded once to dt)
 *   out = x + layer(xn)                          (residual != 0; the sum is
 *         taken in fp32 with the combine, then rounded once)
 *
 * where layer() is the plain entry point's computation (routing included).
 * norm_w is a device array [d] of type dt (bf16 for the MXFP4 layer; bf16
 * norm weights 16-byte aligned); eps must be finite and >= 0.  A NULL block
 * is the plain layer.  With bf16 and more than 16 tokens the norm runs
 * inside the router kernel, which streams the rows anyway and writes the
 * normalised rows to the workspace for the expert stages; fp32 blocks and
 * blocks of at most 16 tokens run a norm kernel first. */
typedef struct {
  const void* norm_w; /* [d] RMSNorm scale; NULL = no norm */
  float eps;          /* RMSNorm epsilon (used when norm_w != NULL) */
  int residual;       /* nonzero: add x to the layer output */
} moe_block;

/* Workspace bytes of a block call (the normalised rows need T * d elements
 * more when block->norm_w != NULL).  Same conventions as
 * moe_ffn_workspace_bytes, which it equals for a NULL block. */
size_t moe_block_workspace_bytes(const moe_block* block, int T, int d, int d_ff, int E, int k,
                                 moe_dtype dt, int grouped, int d_ff_shared);

/* The three layers as blocks: arguments as moe_ffn_forward,
 * moe_ffn_forward_mxfp4 and moe_ffn_forward_grouped, plus `block`.
 * Errors as there; in addition MOE_ERR_INVALID_ARG for a negative or
 * non-finite eps, and MOE_ERR_WORKSPACE when the workspace is smaller than
 * moe_block_workspace_bytes(). */
moe_status moe_block_forward(const moe_block* block, const void* x, const void* router_w, const void* router_b,
                             const void* w_gate, const void* b_gate,
                             const void* w_up, const void* b_up,
                             const void* w_down, const void* b_down,
                             int T, int d, int d_ff, int E, int k, float alpha, float limit,
                             void* out, moe_dtype dt, void* workspace, size_t workspace_bytes,
                             moe_routing_out* routing, hipStream_t stream);

moe_status moe_block_forward_mxfp4(const moe_block* block, const void* x, const void* router_w,
                                   const void* router_b,
                                   const uint8_t* w_gate_codes, const uint8_t* w_gate_scales, const void* b_gate,
                                   const uint8_t* w_up_codes, const uint8_t* w_up_scales, const void* b_up,
                                   const uint8_t* w_down_codes, const uint8_t* w_down_scales, const void* b_down,
                                   int T, int d, int d_ff, int E, int k, float alpha, float limit,
                                   void* out, void* workspace, size_t workspace_bytes,
                                   moe_routing_out* routing, hipStream_t stream);

moe_status moe_block_forward_grouped(const moe_block* block, const void* x, const void* router_w,
                                     const void* router_b, const float* e_score_bias,
                                     const void* w_gate, const void* b_gate,
                                     const void* w_up, const void* b_up,
                                     const void* w_down, const void* b_down,
                                     const void* shared_w_gate, const void* shared_w_up,
                                     const void* shared_w_down, int d_ff_shared,
                                     int T, int d, int d_ff, int E, int k,
                                     int n_group, int topk_group, int norm_topk_prob,
                                     float routed_scaling_factor, moe_score score,
                                     moe_act act, float alpha, float limit,
                                     void* out, moe_dtype dt, void* workspace, size_t workspace_bytes,
                                     moe_routing_out* routing, hipStream_t stream);

/* ---- Affine group-quantized routed experts -------------------------------
 * glm4_moe_lite.go runs quantized experts through GatherQMM on (weight,
 * scales, biases) with the affine mode of quantizationParams: INT4 = 4-bit
 * codes in groups of 32, INT8 = 8-bit codes in groups of 64 (SwitchMLP,
 * supportsGatherQMM, quantizationParams, loadExpertWeight).  The weight is
 *   w[e][n][k] = scales[e][n][k / G] * q[e][n][k] + biases[e][n][k / G]
 * with unsigned codes q in [0, 2^bits).  Layouts (rows, cols) as the dense
 * weights, (d_ff, d) for gate and up, (d, d_ff) for down:
 *   *_q       uint8 [E, rows, cols * bits / 8]: 8 bits one byte per element;
 *             4 bits element 2i in the low nibble, 2i+1 in the high nibble;
 *   *_scales, *_biases  bf16 [E, rows, cols / G].
 * The decoded weight is rounded once to bf16 before the products. */
typedef struct {
  int bits; /* 4 (groups of 32) or 8 (groups of 64) */
  const uint8_t* gate_q; const void* gate_scales; const void* gate_biases;
  const uint8_t* up_q;   const void* up_scales;   const void* up_biases;
  const uint8_t* down_q; const void* down_scales; const void* down_biases;
} moe_affine_experts;

/* The GLM4-MoE-style layer (moe_ffn_forward_grouped's routing, activation,
 * shared expert, expert biases) with affine group-quantized routed experts;
 * x, router, biases, shared expert and out are bf16; `block` as in
 * moe_block_forward_grouped (NULL: the plain layer).  Requires bits 4 or 8,
 * d and d_ff multiples of the group size (MOE_ERR_UNSUPPORTED), every
 * code / scale / bias pointer (MOE_ERR_INVALID_ARG), and the size limits of
 * the MXFP4 layer for the codes (d * d_ff * bits / 8 < 2^32). */
moe_status moe_block_forward_grouped_affine(const moe_block* block, const moe_affine_experts* experts,
                                            const void* x, const void* router_w, const void* router_b,
                                            const float* e_score_bias,
                                            const void* b_gate, const void* b_up, const void* b_down,
                                            const void* shared_w_gate, const void* shared_w_up,
                                            const void* shared_w_down, int d_ff_shared,
                                            int T, int d, int d_ff, int E, int k,
                                            int n_group, int topk_group, int norm_topk_prob,
                                            float routed_scaling_factor, moe_score score,
                                            moe_act act, float alpha, float limit,
                                            void* out, void* workspace, size_t workspace_bytes,
                                            moe_routing_out* routing, hipStream_t stream);

/* ---- No-allocation entry point --------------------------------------------
 * For callers that cannot allocate device memory: work recorded under HIP
 * graph capture, serving loops and harnesses that forbid hipMalloc.
 * moe_ffn_forward_noalloc is moe_ffn_forward without the workspace
 * arguments.  Its workspace is a fixed array in the library's device code of
 * MOE_NOALLOC_SCRATCH_BYTES bytes: the loader gives every GPU the library
 * runs on a copy of its own, held until the process ends.  The call
 * allocates nothing and calls no allocating routine; it runs the same
 * kernels as moe_ffn_forward, on `stream`, on the stream's GPU (the current
 * GPU for the null stream).
 * Limit: a layer whose moe_ffn_workspace_bytes(T, d, d_ff, E, k, dt, 0, 0)
 * exceeds MOE_NOALLOC_SCRATCH_BYTES returns MOE_ERR_WORKSPACE and launches
 * nothing (at d = d_ff = 2880, E = 32, k = 4, bf16: T up to about 1400).
 * Every call on one GPU works in that GPU's single array: calls that can
 * overlap in time on one GPU (on two streams, or from two threads without
 * ordering between their streams) race on it and give wrong results; calls
 * queued on one stream are ordered and safe.  No part of the array needs to
 * start at zero (every kernel writes what a later kernel reads), and a call
 * leaves the previous call's contents in it.  Errors as moe_ffn_forward,
 * plus MOE_ERR_HIP when the array's address cannot be obtained. */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)

moe_status moe_ffn_forward_noalloc(const void* x, const void* router_w, const void* router_b,
                                   const void* w_gate, const void* b_gate,
                                   const void* w_up, const void* b_up,
                                   const void* w_down, const void* b_down,
                                   int T, int d, int d_ff, int E, int k, float alpha, float limit,
                                   void* out, moe_dtype dt, moe_routing_out* routing, hipStream_t stream);

/* Name of a status code (static string). */
const char* moe_status_string(moe_status s);

/* Description of the last error returned on the calling thread (static,
 * thread-local storage; empty after a successful call). */
const char* moe_last_error_detail(void);

/* ---- Opt-in stage timing -------------------------------------------------
 * Stages of one call, in launch order.  A shared expert's products are timed
 * with the gate|up and down stages, except in bf16 calls with more than 16
 * tokens, at most 128 routed experts and no RMSNorm prologue: there its
 * gate|up tiles run in the router's launch and its down tiles in the
 * permutation's, and are timed with those stages. */
typedef enum {
  MOE_STAGE_ROUTE = 0,    /* (block RMSNorm +) router logits + top-k + weights */
  MOE_STAGE_PERMUTE = 1,  /* per-expert counts, prefix sums, stable scatter */
  MOE_STAGE_GATE_UP = 2,  /* grouped gate|up GEMM + bias + activation */
  MOE_STAGE_DOWN = 3,     /* grouped down GEMM + bias */
  MOE_STAGE_COMBINE = 4,  /* weighted gather-reduce back to token order */
  MOE_NUM_STAGES = 5
} moe_stage;

/* Enable (stage_mask != 0) or disable (0) timing of the stages whose bit
 * (1 << moe_stage) is set.  While enabled, every forward call records a HIP
 * event before and after each selected stage on its stream.  Events are
 * created here (not in the forward calls).  Process-wide; not thread-safe. */
moe_status moe_ffn_profile_enable(unsigned stage_mask);

/* Wait for the recorded events, then write, per stage, the summed duration
 * in milliseconds and the number of timed launches since the last read (or
 * enable), and reset the sums.  ms and launches have n_stages entries. */
moe_status moe_ffn_profile_read(double* ms, int* launches, int n_stages);

#ifdef __cplusplus
}
#endif

#endif /* MOE_FFN_H */
