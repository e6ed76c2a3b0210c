"""The MoE-FFN layer workloads this library is tested and measured on.

Each workload fixes the layer's shapes, its routing flavour and the recipe of
its seeded synthetic inputs.  Shapes follow the pages:

* GPT-OSS-20B MoE layer: 32 experts with 4 active per token ("GPT-OSS 20B GGUF
  with MoE CPU Offloading Support", Key Features / Model Specifications); the
  clipped SwiGLU with alpha = 1.702 ("Implementation: Ollama Imagegen GPT OSS",
  Description); router, gate, up and down all carry a bias (MaxText GPT-OSS
  weight mapping, "MoE Router" and "MOE EXPERTS" blocks).
* GLM4-MoE-Lite MoE layer: n_routed_experts / n_shared_experts /
  num_experts_per_tok / routed_scaling_factor / norm_topk_prob / n_group /
  topk_group (glm4_moe_lite.go, Config), SiLU-gated experts without bias
  (glm4_moe_lite.go, SwitchMLP and SharedExperts).

The hidden size d = d_ff = 2880 of the GPT-OSS shapes, the token counts, the
distributions and the MXFP4 scale range are not on the pages; they are the
workload definitions this library is measured on.
"""
from __future__ import annotations

import dataclasses
from typing import Optional


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d: int
    d_ff: int
    E: int
    k: int
    dtype: str                 # "f32" | "bf16" (activations, dense weights, biases, out)
    weights: str = "dense"     # "dense" | "mxfp4" | "mxfp8" | "nvfp4" | "affine4" (groups of 32) | "affine8" (groups of 64)
    # "mxfp8": the expert GEMMs' activation operands are converted to MXFP8
    # (MXFP4 weights on the gfx950 scaled MFMA)
    act_quant: Optional[str] = None
    routing: str = "gptoss"    # "gptoss" (top-k over logits, softmax over selected) | "grouped"
    act: str = "clipped_swiglu"  # "clipped_swiglu" | "silu"
    alpha: float = 1.702
    limit: float = 7.0
    # grouped (GLM) routing
    n_group: int = 1
    topk_group: int = 1
    norm_topk_prob: bool = False
    routed_scaling_factor: float = 1.0
    score: str = "softmax"     # "softmax" | "sigmoid"
    d_ff_shared: int = 0       # 0 = no shared expert
    # MoE block (glm4_moe_lite.go, MoEBlock.Forward after attention):
    # out = x + layer(RMSNorm(x; gamma, norm_eps))
    block: bool = False
    norm_eps: float = 1e-5
    # input recipe
    router_bias: str = "normal"   # "normal" | "zero" | "zipf" | "none"
    expert_bias: bool = True
    bias_std: float = 0.02
    zipf_s: float = 1.1
    mx_scale_exp_lo: int = -8
    mx_scale_exp_hi: int = -2
    seed: int = 0

    @property
    def P(self) -> int:
        """Number of (token, slot) pairs routed to experts."""
        return self.T * self.k

    def scaled(self, T: Optional[int] = None, **kw) -> "Workload":
        """Same layer with another token count (or other overrides)."""
        if T is not None:
            kw["T"] = T
        return dataclasses.replace(self, **kw)


TINY_F32 = Workload(
    name="tiny_fp32_T16_d64_E8_k2", T=16, d=64, d_ff=64, E=8, k=2, dtype="f32",
    router_bias="normal")

GPTOSS_DECODE = Workload(
    name="gptoss20b_decode_T8_d2880_E32_k4_bf16", T=8, d=2880, d_ff=2880, E=32, k=4,
    dtype="bf16", router_bias="zero")

GPTOSS_PREFILL = Workload(
    name="gptoss20b_prefill_T8192_d2880_E32_k4_bf16", T=8192, d=2880, d_ff=2880, E=32, k=4,
    dtype="bf16", router_bias="zipf")

GPTOSS_MXFP4 = Workload(
    name="gptoss20b_mxfp4_T4096_d2880_E32_k4", T=4096, d=2880, d_ff=2880, E=32, k=4,
    dtype="bf16", weights="mxfp4", router_bias="zero")

GLM4_MOE_LITE = Workload(
    name="glm4moelite_T2048_d2048_F1536_E64s1_k6_g8tg4", T=2048, d=2048, d_ff=1536, E=64, k=6,
    dtype="bf16", routing="grouped", act="silu", n_group=8, topk_group=4,
    norm_topk_prob=True, routed_scaling_factor=1.8, score="softmax", d_ff_shared=1536,
    router_bias="none", expert_bias=False)

ALL = (TINY_F32, GPTOSS_DECODE, GPTOSS_PREFILL, GPTOSS_MXFP4, GLM4_MOE_LITE)

# GLM4-MoE-Lite with affine group-quantized routed experts (glm4_moe_lite.go:
# SwitchMLP through GatherQMM; quantizationParams INT4 = groups of 32 x 4 bits,
# INT8 = groups of 64 x 8 bits, mode affine).  The shared expert stays bf16.
GLM4_MOE_LITE_INT4 = GLM4_MOE_LITE.scaled(name="glm4moelite_int4g32_T2048_d2048_F1536_E64s1_k6_g8tg4",
                                          weights="affine4")
GLM4_MOE_LITE_INT8 = GLM4_MOE_LITE.scaled(name="glm4moelite_int8g64_T2048_d2048_F1536_E64s1_k6_g8tg4",
                                          weights="affine8")
QUANTIZED = (GLM4_MOE_LITE_INT4, GLM4_MOE_LITE_INT8)

# The same layers as MoE blocks: RMSNorm in front, residual added
# (glm4_moe_lite.go, MoEBlock.Forward; Config.RMSNormEps).
GLM4_MOE_LITE_BLOCK = GLM4_MOE_LITE.scaled(name="glm4moelite_block_T2048_d2048_F1536_E64s1_k6_g8tg4",
                                           block=True)
GPTOSS_DECODE_BLOCK = GPTOSS_DECODE.scaled(name="gptoss20b_block_decode_T8_d2880_E32_k4_bf16", block=True)
# A dense block of the first_k_dense_replace layers (glm4_moe_lite.go, DenseBlock
# and DenseMLP: down(silu(gate(x)) * up(x)), no router) is the E = k = 1 case
# of the grouped layer: one expert, softmax over one logit = weight 1.  The
# dense intermediate size (8192 here) is not on the pages.
GLM4_DENSE_BLOCK = Workload(
    name="glm4_dense_block_T2048_d2048_F8192", T=2048, d=2048, d_ff=8192, E=1, k=1,
    dtype="bf16", routing="grouped", act="silu", n_group=1, topk_group=1, norm_topk_prob=False,
    routed_scaling_factor=1.0, score="softmax", router_bias="none", expert_bias=False, block=True)
BLOCKS = (GPTOSS_DECODE_BLOCK, GLM4_MOE_LITE_BLOCK, GLM4_DENSE_BLOCK)

# The MXFP4 layer with MXFP8 activations (OCP MX E4M3, groups of 32, the
# MXFP8 mode of glm4_moe_lite.go quantizationParams) on the scaled MFMA.
GPTOSS_MXFP4_MX8 = GPTOSS_MXFP4.scaled(name="gptoss20b_mxfp4_mxfp8act_T4096_d2880_E32_k4", act_quant="mxfp8")
# MXFP8 expert weights (E4M3 codes, e8m0 scale per 32) with MXFP8 activations.
# Codes are uniform over the finite E4M3 codes (root mean square ~87), so the
# scale exponents -16 .. -12 keep the gate and up pre-activations O(1).
GPTOSS_MXFP8_MX8 = GPTOSS_MXFP4.scaled(name="gptoss20b_mxfp8w_mxfp8act_T4096_d2880_E32_k4", weights="mxfp8",
                                       act_quant="mxfp8", mx_scale_exp_lo=-16, mx_scale_exp_hi=-12)
MX_ACT = (GPTOSS_MXFP4_MX8, GPTOSS_MXFP8_MX8)
# The MXFP4 layer at decode (8 tokens): weight streaming of the 4.25-bit experts.
GPTOSS_MXFP4_DECODE = GPTOSS_MXFP4.scaled(T=8, name="gptoss20b_mxfp4_decode_T8_d2880_E32_k4")
# NVFP4 expert weights (e2m1 codes, an E4M3 scale per 16, a tensor scale),
# decoded to bf16 in registers (quantizationParams: NVFP4 = groups of 16, 4 bits).
GPTOSS_NVFP4 = GPTOSS_MXFP4.scaled(name="gptoss20b_nvfp4_T4096_d2880_E32_k4", weights="nvfp4")

BY_NAME = {w.name: w for w in ALL + BLOCKS + QUANTIZED + MX_ACT + (GPTOSS_NVFP4, GPTOSS_MXFP4_DECODE)}
