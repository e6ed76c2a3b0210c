"""CPU oracle of one Mixture-of-Experts feed-forward layer, in float64.

TEST INFRASTRUCTURE ONLY.  This module is the plain, slow reference that the
GPU library is checked against.  Only the test suite, the package smoke check
and the benchmark's CPU-baseline leg may import or run it; the library itself
never does, and this module imports nothing from the library.

Sources (cited by page title and section; the pages are web pages about the
MoE layers of GPT-OSS and GLM4-MoE-Lite):

  [GPTOSS]  "Implementation:Ollama Ollama Imagegen GPT OSS" -- Description and
            Signature (clipped SwiGLU, alpha = 1.702, Config fields).
  [GGUF]    "GPT-OSS 20B GGUF with MoE CPU Offloading Support" -- Key Features
            and Model Specifications (32 experts / 4 active, MXFP4 experts).
  [MAXTEXT] MaxText "weight_mapping/gpt_oss" module -- the "MoE Router" and
            "MOE EXPERTS" blocks of to_hf_mapping (router kernel + bias,
            gate_proj / up_proj kernels + biases, mlp2 weight + bias).
  [GLM]     "x/models/glm4_moe_lite/glm4_moe_lite.go" -- Config, DenseMLP,
            MoEGate.Forward, SwitchMLP.Forward, SharedExperts.Forward,
            MoE.Forward.
  [OCP-MX]  OCP Microscaling Formats (MX) v1.0 specification (not on the
            pages; it defines the e2m1 element and e8m0 scale the MXFP4 name
            on [GGUF] refers to).
  [MXFP8]   the same page's quantizationParams names MXFP8 (groups of 32,
            8 bits) as a quantization mode; [OCP-MX] defines the E4M3
            element, the e8m0 scale and the conversion of a block of 32
            values (scale exponent = floor(log2 of the block's largest
            magnitude) - 8, elements rounded to nearest-even E4M3).
  [NVFP4]   the same page's quantizationParams names NVFP4 (groups of 16, 4
            bits, mode nvfp4) without its layout; read as the published
            NVFP4 definition: e2m1 elements, an E4M3 scale per block of 16
            and one fp32 scale per tensor.
  [GLM-Q]   the same glm4_moe_lite.go page on quantized experts:
            SwitchMLP (GatherQMM with weight, scales and biases, group size,
            bits, mode), supportsGatherQMM (affine, 4 or 8 bits),
            quantizationParams (INT4: groups of 32, 4 bits, affine; INT8:
            groups of 64, 8 bits, affine), loadExpertWeight.

Readings taken where the pages are silent or disagree (each is listed with its
reason in the design notes of this repository):
  * GPT-OSS routing: top-k of the raw router logits, weights = softmax over the
    k selected logits ([MAXTEXT] shows only an affine router; [GPTOSS] does
    not describe it).
  * Ordering and ties: experts ordered by (score descending, index ascending);
    an exact tie goes to the lower index.
  * Clipped SwiGLU: g' = clip(g, 0, limit), u' = clip(u, -limit, limit),
    h = g' * sigmoid(alpha * g') * u'  ([GPTOSS] Description, taken literally).
  * Biases are added by each Linear before the activation; the down bias is
    inside each expert's output, before the routing weight.
  * GLM grouped routing: scores s = softmax(logits) over all experts (or
    sigmoid, as [GLM] MoEGate.Forward computes); the group score is the
    largest selection score in each contiguous group of E/n_group experts;
    topk_group groups are kept (ties to the lower group index); top-k is taken
    among the kept experts on the selection score (score + correction bias);
    weights are the unbiased scores of the chosen experts, renormalised when
    k > 1 and norm_topk_prob, then multiplied by routed_scaling_factor.
  * The shared expert is a SiLU-gated MLP without bias, weight 1, added after
    the routed sum ([GLM] SharedExperts.Forward, MoE.Forward).
  * Permutation: pairs p = t*k + j sorted by (expert, p) (a stable sort).
  * MoE block ([GLM] MoEBlock.Forward, the half after attention): the layer
    sees RMSNorm(x) = x / sqrt(mean(x^2) + eps) * gamma (nn.RMSNorm with
    Config.RMSNormEps; the pages do not print its formula, this is the plain
    definition) and its output is added to x.  The norm's output is an array
    of the layer's element type (MLX arrays keep their dtype), so the layer
    sees it rounded to nearest-even bf16 (fp32).
  * MXFP8 activations (act_quant = "mxfp8", for MXFP4 experts on the
    gfx950 scaled MFMA): the rows entering each expert and the hidden
    activation h, as a bf16 array, are converted to MXFP8 by the [OCP-MX]
    block conversion along the input dimension; elements beyond the E4M3
    range saturate to +-448; a block holding a NaN or an infinity gets the
    NaN scale (255); an all-zero block gets scale byte 0.
"""
from __future__ import annotations

import itertools
from typing import Optional

import numpy as np

# ----------------------------------------------------------------------------
# Decoding of stored inputs into float64.


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64.  bf16 is the top half of an
    IEEE binary32, so widening is exact."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def to_f64(a: Optional[np.ndarray], dtype: str) -> Optional[np.ndarray]:
    """Stored array (bf16 bits or float32) -> float64; None stays None."""
    if a is None:
        return None
    if dtype == "bf16":
        return bf16_to_f64(a)
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


# [OCP-MX] FP4 E2M1: 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit.
# Magnitudes of codes 0..7; codes 8..15 are the same with the sign bit set.
E2M1_MAGNITUDE = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


def e2m1_value(code: np.ndarray) -> np.ndarray:
    """Value of a 4-bit e2m1 code ([OCP-MX] FP4 element)."""
    code = np.asarray(code, dtype=np.uint8)
    mag = E2M1_MAGNITUDE[code & 7]
    return np.where(code & 8, -mag, mag)


def e8m0_value(scale: np.ndarray) -> np.ndarray:
    """Value of an e8m0 block scale: 2**(byte - 127); byte 255 is NaN ([OCP-MX])."""
    s = np.asarray(scale, dtype=np.int64)
    v = np.ldexp(1.0, (s - 127).astype(np.int32))
    return np.where(s == 255, np.nan, v)


def e4m3_value(code: np.ndarray) -> np.ndarray:
    """Value of an OCP E4M3 code ([OCP-MX]): bit 7 sign, bits 6..3 exponent
    (bias 7), bits 2..0 mantissa; exponent 0 is subnormal (m/8 * 2^-6);
    S.1111.111 is NaN; there are no infinities."""
    c = np.asarray(code, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    v = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.ldexp(1.0, (e - 7).astype(np.int32)))
    return np.where((c & 0x7F) == 0x7F, np.nan, sign * v)


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """Nearest E4M3 code of finite float64 values, ties to even; magnitudes
    at or above the largest normal, 448, give 448 (saturation).  The sign
    bit is v's sign bit (-0 gives 0x80)."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    # subnormal range (a < 2^-6): steps of 2^-9, codes 0..8 (8 is 2^-6)
    q_sub = np.round(a * 512.0)                    # numpy rounds halves to even
    # normal range: a = f 2^x with f in [0.5, 1); 16 f rounded gives the
    # implicit bit and 3 mantissa bits (16 carries into the exponent)
    f, x = np.frexp(a)
    r = np.round(f * 16.0)
    q_norm = (x - 1 + 7) * 8 + (r - 8)
    mag = np.where(a >= 448.0, 0x7E, np.where(a < 2.0 ** -6, q_sub, q_norm))
    return (mag.astype(np.int64) | np.where(np.signbit(v), 0x80, 0)).astype(np.uint8)


def mxfp8_quantize(v: np.ndarray):
    """MXFP8 conversion of float64 rows [n, K] (K % 32 == 0) in blocks of 32
    consecutive elements ([OCP-MX] conversion; [MXFP8] group of 32):
        s = floor(log2(max |v_i|)) - 8   (8 = the E4M3 largest exponent),
        clamped to the e8m0 range [-127, 127];
        codes = e4m3_encode(v_i / 2^s), scale byte = s + 127.
    An all-zero block gets scale byte 0 (zero codes); a block with a NaN or an
    infinity gets scale byte 255 (NaN) and zero codes.
    Returns (codes uint8 [n, K], scales uint8 [n, K/32])."""
    v = np.asarray(v, dtype=np.float64)
    n, K = v.shape
    b = v.reshape(n, K // 32, 32)
    amax = np.max(np.abs(np.where(np.isfinite(b), b, 0.0)), axis=-1)
    bad = ~np.all(np.isfinite(b), axis=-1)
    _, x = np.frexp(amax)                              # floor(log2 amax) = x - 1 for amax > 0
    s = np.clip(x - 1 - 8, -127, 127)
    s = np.where(amax > 0, s, -127)
    scaled = np.where(np.isfinite(b), b, 0.0) / np.ldexp(1.0, s.astype(np.int32))[..., None]
    codes = e4m3_encode(scaled)
    codes = np.where(bad[..., None], np.uint8(0), codes)
    scales = np.where(bad, 255, s + 127).astype(np.uint8)
    return codes.reshape(n, K), scales


def mxfp8_dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Values of MXFP8 rows: e4m3_value(code) * 2^(scale - 127) per block of
    32 (scale byte 255: NaN)."""
    codes = np.asarray(codes)
    n, K = codes.shape
    return (e4m3_value(codes).reshape(n, K // 32, 32) * e8m0_value(scales)[..., None]).reshape(n, K)


def mxfp8_round(v: np.ndarray) -> np.ndarray:
    """v as the MXFP8 values it converts to (quantize, then dequantize)."""
    return mxfp8_dequantize(*mxfp8_quantize(v))


def nvfp4_decode(codes: np.ndarray, scales: np.ndarray, tensor_scale: float) -> np.ndarray:
    """Decode one NVFP4 matrix ([NVFP4]): codes uint8 [rows, cols/2] (element 2i
    in the low nibble), scales uint8 [rows, cols/16] of E4M3 codes, one per 16
    consecutive elements of a row, and a float tensor scale:
        w[r, c] = e2m1(code[r, c]) * e4m3(scale[r, c // 16]) * tensor_scale."""
    codes = np.asarray(codes, dtype=np.uint8)
    rows, half = codes.shape
    elem = np.empty((rows, 2 * half), dtype=np.float64)
    elem[:, 0::2] = e2m1_value(codes & 0x0F)
    elem[:, 1::2] = e2m1_value(codes >> 4)
    sc = np.repeat(e4m3_value(scales), 16, axis=1)
    assert sc.shape == elem.shape
    return elem * sc * float(tensor_scale)


def affine_decode(q: np.ndarray, scales: np.ndarray, biases: np.ndarray, bits: int, group: int) -> np.ndarray:
    """Decode one affine group-quantized matrix ([GLM-Q]; the pages name the
    mode, the bits, the group size and the scale / bias arrays but print no
    formula -- this is the plain affine reading):
        w[r, c] = scales[r, c // group] * q[r, c] + biases[r, c // group]
    with unsigned codes q in [0, 2^bits).  q is stored as uint8 [rows,
    cols * bits / 8]: 8 bits one byte per element; 4 bits element 2i in the
    low nibble and 2i+1 in the high nibble.  scales and biases are float64
    [rows, cols / group]."""
    q = np.asarray(q, dtype=np.uint8)
    if bits == 8:
        elem = q.astype(np.float64)
    elif bits == 4:
        rows, half = q.shape
        elem = np.empty((rows, 2 * half), dtype=np.float64)
        elem[:, 0::2] = q & 0x0F
        elem[:, 1::2] = q >> 4
    else:
        raise ValueError(bits)
    s = np.repeat(np.asarray(scales, dtype=np.float64), group, axis=1)
    b = np.repeat(np.asarray(biases, dtype=np.float64), group, axis=1)
    assert s.shape == elem.shape
    return s * elem + b


def mxfp4_decode(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Decode one MXFP4 matrix: codes uint8 [rows, cols/2] (element 2i in the
    low nibble, 2i+1 in the high nibble), scales uint8 [rows, cols/32], one per
    32 consecutive elements of a row.  Returns float64 [rows, cols]."""
    codes = np.asarray(codes, dtype=np.uint8)
    rows, half = codes.shape
    cols = 2 * half
    elem = np.empty((rows, cols), dtype=np.uint8)
    elem[:, 0::2] = codes & 0x0F
    elem[:, 1::2] = codes >> 4
    blk_scale = np.repeat(e8m0_value(scales), 32, axis=1)
    assert blk_scale.shape == (rows, cols)
    return e2m1_value(elem) * blk_scale


# ----------------------------------------------------------------------------
# Router.


def router_logits(x: np.ndarray, w_router: np.ndarray, b_router: Optional[np.ndarray]) -> np.ndarray:
    """l[t, e] = sum_i x[t, i] * Wr[e, i] + br[e]  -- the router is an affine map
    from the hidden size to one logit per expert ([MAXTEXT] "MoE Router": a
    kernel and a bias; [GLM] MoEGate.Forward: Gate Linear)."""
    l = x @ w_router.T
    if b_router is not None:
        l = l + b_router[None, :]
    return l


def order_desc(v: np.ndarray) -> np.ndarray:
    """Indices of each row of v ordered by (value descending, index ascending)."""
    return np.argsort(-v, axis=-1, kind="stable")


def gptoss_route(logits: np.ndarray, k: int):
    """Top-k experts of each token and their weights.

    Selection: the k largest logits (ties to the lower expert index).
    Weights: softmax over the k selected logits.
    Returns idx int64 [T, k] in selection order, w float64 [T, k]."""
    idx = order_desc(logits)[:, :k]
    sel = np.take_along_axis(logits, idx, axis=1)
    m = sel[:, :1]
    ex = np.exp(sel - m)
    w = ex / ex.sum(axis=1, keepdims=True)
    return idx, w


def sigmoid(z: np.ndarray) -> np.ndarray:
    """Logistic function 1 / (1 + exp(-z)), evaluated without overflow."""
    z = np.asarray(z, dtype=np.float64)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    out[~pos] = ez / (1.0 + ez)
    return out


def softmax(z: np.ndarray) -> np.ndarray:
    """Softmax over the last axis (max-subtracted)."""
    m = z.max(axis=-1, keepdims=True)
    ex = np.exp(z - m)
    return ex / ex.sum(axis=-1, keepdims=True)


def grouped_route(logits: np.ndarray, k: int, n_group: int, topk_group: int,
                  norm_topk_prob: bool, routed_scaling_factor: float,
                  score: str = "softmax", e_score_bias: Optional[np.ndarray] = None):
    """Group-limited routing of GLM4-MoE style ([GLM] Config fields n_group /
    topk_group / norm_topk_prob / routed_scaling_factor; [GLM] MoEGate.Forward).

    1. s = softmax(l) over all experts, or sigmoid(l) ([GLM] MoEGate.Forward).
    2. s' = s + e_score_bias when a correction bias is given (selection only).
    3. Experts form n_group contiguous groups of E/n_group; group score =
       max of s' over the group; keep the topk_group best groups.
    4. idx = the k best experts by s' among the kept groups.
    5. w = s[idx]; if k > 1 and norm_topk_prob: w /= sum(w); w *= rsf.
    Returns idx int64 [T, k], w float64 [T, k]."""
    T, E = logits.shape
    assert E % n_group == 0 and 1 <= topk_group <= n_group
    s = softmax(logits) if score == "softmax" else sigmoid(logits)
    s_sel = s + e_score_bias[None, :] if e_score_bias is not None else s
    gsize = E // n_group
    group_score = s_sel.reshape(T, n_group, gsize).max(axis=2)
    kept_groups = order_desc(group_score)[:, :topk_group]
    allowed = np.zeros((T, n_group), dtype=bool)
    np.put_along_axis(allowed, kept_groups, True, axis=1)
    allowed_e = np.repeat(allowed, gsize, axis=1)
    cand = np.where(allowed_e, s_sel, -np.inf)
    idx = order_desc(cand)[:, :k]
    assert np.all(np.take_along_axis(allowed_e, idx, axis=1)), "k exceeds the kept experts"
    w = np.take_along_axis(s, idx, axis=1)
    if k > 1 and norm_topk_prob:
        w = w / w.sum(axis=1, keepdims=True)
    w = w * routed_scaling_factor
    return idx, w


# ----------------------------------------------------------------------------
# Expert MLP.


def clipped_swiglu(g: np.ndarray, u: np.ndarray, alpha: float, limit: float) -> np.ndarray:
    """GPT-OSS activation ([GPTOSS] Description): gate clipped to [0, limit],
    up clipped to [-limit, limit], sigmoid scaled by alpha:
        h = g' * sigmoid(alpha * g') * u'."""
    gc = np.minimum(np.maximum(g, 0.0), limit)
    uc = np.minimum(np.maximum(u, -limit), limit)
    return gc * sigmoid(alpha * gc) * uc


def silu_glu(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """SiLU-gated product ([GLM] DenseMLP / SwitchMLP / SharedExperts):
        h = silu(g) * u = g * sigmoid(g) * u."""
    return g * sigmoid(g) * u


def activation(g, u, act: str, alpha: float, limit: float):
    if act == "clipped_swiglu":
        return clipped_swiglu(g, u, alpha, limit)
    if act == "silu":
        return silu_glu(g, u)
    raise ValueError(act)


def expert_mlp(X: np.ndarray, Wg, bg, Wu, bu, Wd, bd, act: str, alpha: float, limit: float,
               act_quant: Optional[str] = None) -> np.ndarray:
    """One expert on the rows of X [n, d]:
        g = X Wg^T + bg ; u = X Wu^T + bu ; h = act(g, u) ; y = h Wd^T + bd
    ([MAXTEXT] "MOE EXPERTS": separate gate_proj / up_proj kernels and biases,
    mlp2 weight and bias; [GLM] SwitchMLP.Forward: gate, up, activation, down).
    act_quant "mxfp8": X and the bf16 array h enter their products as MXFP8
    values (mxfp8_round)."""
    if act_quant == "mxfp8":
        X = mxfp8_round(X)
    elif act_quant is not None:
        raise ValueError(act_quant)
    g = X @ Wg.T
    u = X @ Wu.T
    if bg is not None:
        g = g + bg[None, :]
    if bu is not None:
        u = u + bu[None, :]
    h = activation(g, u, act, alpha, limit)
    if act_quant == "mxfp8":
        h = mxfp8_round(round_bf16(h))
    y = h @ Wd.T
    if bd is not None:
        y = y + bd[None, :]
    return y


class ExpertWeights:
    """Access to one layer's stacked expert weights, decoded to float64 per expert.

    `arrays` holds the stored inputs: w_gate/w_up/w_down (bf16 bits or f32) or
    their MXFP4 / MXFP8 (codes, scales) pairs or affine (codes, scales,
    biases), and b_gate/b_up/b_down (or None)."""

    def __init__(self, arrays: dict, dtype: str, weights: str):
        self.a = arrays
        self.dtype = dtype
        self.weights = weights

    def _mat(self, name: str, e: int) -> np.ndarray:
        if self.weights == "mxfp4":
            return mxfp4_decode(self.a[name + "_codes"][e], self.a[name + "_scales"][e])
        if self.weights == "mxfp8":
            return mxfp8_dequantize(self.a[name + "_codes"][e], self.a[name + "_scales"][e])
        if self.weights == "nvfp4":
            return nvfp4_decode(self.a[name + "_codes"][e], self.a[name + "_scales"][e],
                                float(self.a[name + "_tensor_scale"]))
        if self.weights in ("affine4", "affine8"):
            bits = 4 if self.weights == "affine4" else 8
            group = 32 if bits == 4 else 64
            return affine_decode(self.a[name + "_q"][e], to_f64(self.a[name + "_qscales"][e], self.dtype),
                                 to_f64(self.a[name + "_qbiases"][e], self.dtype), bits, group)
        return to_f64(self.a[name][e], self.dtype)

    def _vec(self, name: str, e: int):
        b = self.a.get(name)
        return None if b is None else to_f64(b[e], self.dtype)

    def expert(self, e: int):
        return (self._mat("w_gate", e), self._vec("b_gate", e),
                self._mat("w_up", e), self._vec("b_up", e),
                self._mat("w_down", e), self._vec("b_down", e))

    def shared(self):
        if self.a.get("shared_w_gate") is None:
            return None
        return (to_f64(self.a["shared_w_gate"], self.dtype), None,
                to_f64(self.a["shared_w_up"], self.dtype), None,
                to_f64(self.a["shared_w_down"], self.dtype), None)


# ----------------------------------------------------------------------------
# MoE block: RMSNorm before the layer, residual after it.


def rms_norm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis ([GLM] MoEBlock.Forward applies
    PostAttentionLayerNorm, an nn.RMSNorm with Config.RMSNormEps, to the MoE
    input):  y = x / sqrt(mean(x^2) + eps) * gamma."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * gamma


def round_bf16(v: np.ndarray) -> np.ndarray:
    """float64 -> nearest bfloat16 value (8 significant bits), ties to even,
    rounded once from float64 (no float32 step).  For finite values in the
    normal range of bf16 (all this oracle rounds)."""
    m, e = np.frexp(np.asarray(v, dtype=np.float64))   # v = m 2^e, 0.5 <= |m| < 1
    return np.ldexp(np.round(m * 256.0), e - 8)        # numpy rounds halves to even


def round_to(v: np.ndarray, dtype: str) -> np.ndarray:
    """Nearest value of the element type (ties to even), as float64."""
    if dtype == "bf16":
        return round_bf16(v)
    return np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float64)


def layer_input(arrays: dict, cfg: dict, tokens: Optional[np.ndarray] = None) -> np.ndarray:
    """The rows the MoE layer works on, float64: x, or for a block
    (cfg["block"]) RMSNorm(x) with the block's gamma (arrays["norm_w"]),
    rounded to the layer's element type."""
    dt = cfg["dtype"]
    x = to_f64(arrays["x"], dt)
    if tokens is not None:
        x = x[tokens]
    if cfg.get("block"):
        x = round_to(rms_norm(x, to_f64(arrays["norm_w"], dt), float(cfg["norm_eps"])), dt)
    return x


# ----------------------------------------------------------------------------
# Routing of a whole layer, permutation, and the layer forward.


def route(arrays: dict, cfg: dict, tokens: Optional[np.ndarray] = None):
    """Router logits and (idx, w) for the given tokens (all tokens if None).

    cfg keys: dtype, k, routing ("gptoss" | "grouped"); for grouped routing
    also n_group, topk_group, norm_topk_prob, routed_scaling_factor, score;
    optional e_score_bias (float array [E]); block and norm_eps for a MoE
    block (the router sees RMSNorm(x))."""
    dt = cfg["dtype"]
    x = layer_input(arrays, cfg, tokens)
    l = router_logits(x, to_f64(arrays["router_w"], dt), to_f64(arrays.get("router_b"), dt))
    if cfg.get("routing", "gptoss") == "gptoss":
        idx, w = gptoss_route(l, cfg["k"])
    else:
        eb = cfg.get("e_score_bias")
        idx, w = grouped_route(l, cfg["k"], cfg["n_group"], cfg["topk_group"],
                               bool(cfg["norm_topk_prob"]), float(cfg["routed_scaling_factor"]),
                               cfg.get("score", "softmax"),
                               None if eb is None else np.asarray(eb, dtype=np.float64))
    return l, idx, w


def permutation(idx: np.ndarray, E: int):
    """Order in which the (token, slot) pairs visit the experts ([GLM]
    SwitchMLP.Forward: flatten the [T, k] indices, argsort, and the inverse
    argsort to restore token order).

    Pair p = t*k + j.  sorted_pair lists the pairs of expert 0 in increasing p,
    then those of expert 1, and so on; pos is its inverse (pos[sorted_pair[r]] = r).
    counts[e] = pairs routed to e; offsets = exclusive prefix sum (E+1 entries)."""
    flat = np.asarray(idx).reshape(-1)
    counts = np.zeros(E, dtype=np.int64)
    sorted_pair = []
    for e in range(E):
        members = np.nonzero(flat == e)[0]       # increasing p
        counts[e] = members.size
        sorted_pair.append(members)
    sorted_pair = np.concatenate(sorted_pair) if sorted_pair else np.zeros(0, np.int64)
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    pos = np.empty_like(sorted_pair)
    pos[sorted_pair] = np.arange(sorted_pair.size)
    return counts, offsets, sorted_pair, pos


def experts_forward(arrays: dict, cfg: dict, idx: np.ndarray, w: np.ndarray,
                    tokens: Optional[np.ndarray] = None) -> np.ndarray:
    """Routed experts and combine for the given tokens with the given routing:

        out[t] = sum_{j = 0..k-1} w[t, j] * FFN_{idx[t, j]}(x_t)   (+ shared(x_t))

    ([GLM] MoE.Forward: sum over the k expert outputs weighted by the gate
    scores, then the shared experts added).  idx/w are [len(tokens), k].
    For a MoE block (cfg["block"]) the experts see RMSNorm(x) and the result
    is added to x ([GLM] MoEBlock.Forward)."""
    dt = cfg["dtype"]
    x = layer_input(arrays, cfg, tokens)
    n, k = idx.shape
    W = ExpertWeights(arrays, dt, cfg.get("weights", "dense"))
    act, alpha, limit = cfg.get("act", "clipped_swiglu"), cfg.get("alpha", 1.702), cfg.get("limit", 7.0)
    y = np.zeros((n, k, x.shape[1]), dtype=np.float64)
    for e in np.unique(idx):
        t_sel, j_sel = np.nonzero(idx == e)
        y[t_sel, j_sel] = expert_mlp(x[t_sel], *W.expert(int(e)), act, alpha, limit, cfg.get("act_quant"))
    out = np.zeros((n, x.shape[1]), dtype=np.float64)
    for j in range(k):
        out += w[:, j:j + 1] * y[:, j]
    sh = W.shared()
    if sh is not None:
        out += expert_mlp(x, *sh, "silu", 0.0, 0.0)
    if cfg.get("block"):
        x_in = to_f64(arrays["x"], dt)
        out = out + (x_in if tokens is None else x_in[tokens])
    return out


def experts_forward_from_h(arrays: dict, cfg: dict, idx: np.ndarray, w: np.ndarray,
                           h: np.ndarray) -> np.ndarray:
    """The second half of the routed layer from given hidden rows:

        out[t] = sum_{j = 0..k-1} w[t, j] * (h[t, j] Wd[idx[t, j]]^T + bd[idx[t, j]])

    ([GLM] SwitchMLP.Forward: the down product of each expert's hidden rows;
    [GLM] MoE.Forward: the weighted sum over the k slots).  h is float64
    [n, k, d_ff], the values the down product consumes (for MXFP8 activations,
    the dequantized E4M3 codes).  Layers with a shared expert or a MoE block
    are not handled here."""
    assert cfg.get("block") is None or not cfg.get("block")
    W = ExpertWeights(arrays, cfg["dtype"], cfg.get("weights", "dense"))
    assert W.shared() is None
    n, k = idx.shape
    Wd0 = W.expert(int(idx.flat[0]))[4] if idx.size else None
    d = Wd0.shape[0] if Wd0 is not None else 0
    y = np.zeros((n, k, d), dtype=np.float64)
    for e in np.unique(idx):
        t_sel, j_sel = np.nonzero(idx == e)
        _, _, _, _, Wd, bd = W.expert(int(e))
        ye = h[t_sel, j_sel] @ Wd.T
        if bd is not None:
            ye = ye + bd[None, :]
        y[t_sel, j_sel] = ye
    out = np.zeros((n, d), dtype=np.float64)
    for j in range(k):
        out += w[:, j:j + 1] * y[:, j]
    return out


def moe_layer(arrays: dict, cfg: dict, tokens: Optional[np.ndarray] = None) -> dict:
    """Whole MoE-FFN layer for the given tokens: routing, experts, combine.
    Returns dict(out, logits, idx, w), all float64 / int64."""
    l, idx, w = route(arrays, cfg, tokens)
    out = experts_forward(arrays, cfg, idx, w, tokens)
    return {"out": out, "logits": l, "idx": idx, "w": w}


def forced_weights(logits: np.ndarray, idx: np.ndarray, cfg: dict) -> np.ndarray:
    """Routing weights of a given expert choice (used for tokens whose choice is
    a near-tie, so that the output can be checked for the choice actually made)."""
    l = np.asarray(logits, dtype=np.float64)
    if cfg.get("routing", "gptoss") == "gptoss":
        sel = np.take_along_axis(l, idx, axis=1)
        ex = np.exp(sel - sel.max(axis=1, keepdims=True))
        return ex / ex.sum(axis=1, keepdims=True)
    s = softmax(l) if cfg.get("score", "softmax") == "softmax" else sigmoid(l)
    w = np.take_along_axis(s, idx, axis=1)
    if idx.shape[1] > 1 and cfg["norm_topk_prob"]:
        w = w / w.sum(axis=1, keepdims=True)
    return w * float(cfg["routed_scaling_factor"])


# ----------------------------------------------------------------------------
# Decision margins (how close a token's expert choice is to a tie).


def selection_values(logits: np.ndarray, cfg: dict) -> np.ndarray:
    """The values a token's expert choice ranks ([GLM] MoEGate.Forward: the
    choice is made on the scores plus the correction bias when one is given).
    GPT-OSS routing and grouped routing without a correction bias rank the
    logits themselves: softmax and sigmoid are increasing in the logit, so the
    order of the experts, and of the group maxima, is that of the logits.
    With a correction bias the ranked values are s + e_score_bias."""
    l = np.asarray(logits, dtype=np.float64)
    if cfg.get("routing", "gptoss") == "grouped" and cfg.get("e_score_bias") is not None:
        s = softmax(l) if cfg.get("score", "softmax") == "softmax" else sigmoid(l)
        return s + np.asarray(cfg["e_score_bias"], dtype=np.float64)[None, :]
    return l


def route_margins(logits: np.ndarray, cfg: dict):
    """Per-token margins of the routing decision in the space where it is made
    (selection_values).

    Returns (boundary, inner): boundary = gap between the last selected and the
    best unselected candidate (for grouped routing also the gap between the
    topk_group-th and the next group score, whichever is smaller); inner =
    smallest gap between consecutive selected experts (decides their order
    only)."""
    l = selection_values(logits, cfg)
    T, E = l.shape
    k = cfg["k"]
    if cfg.get("routing", "gptoss") == "grouped":
        ng, tg = cfg["n_group"], cfg["topk_group"]
        gs = E // ng
        G = l.reshape(T, ng, gs).max(axis=2)
        Gs = -np.sort(-G, axis=1)
        gmargin = Gs[:, tg - 1] - Gs[:, tg] if tg < ng else np.full(T, np.inf)
        kept = order_desc(G)[:, :tg]
        allowed = np.zeros((T, ng), dtype=bool)
        np.put_along_axis(allowed, kept, True, axis=1)
        cand = np.where(np.repeat(allowed, gs, axis=1), l, -np.inf)
    else:
        gmargin = np.full(T, np.inf)
        cand = l
    srt = -np.sort(-cand, axis=1)
    boundary = srt[:, k - 1] - srt[:, k] if k < E else np.full(T, np.inf)
    boundary = np.where(np.isfinite(boundary), boundary, np.inf)
    boundary = np.minimum(boundary, gmargin)
    inner = np.min(srt[:, :k - 1] - srt[:, 1:k], axis=1) if k > 1 else np.full(T, np.inf)
    return boundary, inner


# ----------------------------------------------------------------------------
# Brute-force forms used to pin the oracle on tiny inputs.


def topk_bruteforce(logits_row: np.ndarray, k: int) -> tuple:
    """The k-subset of experts with the largest logit sum (exhaustive)."""
    E = logits_row.shape[0]
    best, best_set = -np.inf, None
    for sub in itertools.combinations(range(E), k):
        s = float(np.sum(logits_row[list(sub)]))
        if s > best:
            best, best_set = s, sub
    return best_set
