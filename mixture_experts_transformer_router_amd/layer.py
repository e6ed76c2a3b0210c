"""Run a described workload through the C ABI: move generated arrays to the
device as torch tensors and call the matching entry point (marshalling only)."""
from __future__ import annotations

import numpy as np
import torch

from . import moe_ffn
from .workloads import Workload


def to_device(arrays: dict, device="cuda") -> dict:
    """numpy arrays (bf16 as uint16 bits) -> device tensors (bf16 / f32 / uint8)."""
    out = {}
    for key, a in arrays.items():
        if a is None:
            out[key] = None
        elif np.ndim(a) == 0:
            out[key] = float(a)        # a scalar (NVFP4 tensor scale) stays on the host
        elif a.dtype == np.uint16:
            out[key] = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
        else:
            out[key] = torch.from_numpy(np.ascontiguousarray(a)).to(device)
    return out


def block_of(w: Workload, t: dict):
    """The moe_block of a block workload (None for a plain layer)."""
    return moe_ffn.make_block(t["norm_w"], w.norm_eps, True) if w.block else None


def workspace_for(w: Workload, device="cuda") -> torch.Tensor:
    dt = moe_ffn.MOE_F32 if w.dtype == "f32" else moe_ffn.MOE_BF16
    blk = moe_ffn.MoeBlock(1, w.norm_eps, 1) if w.block else None  # sizes only
    if w.act_quant == "mxfp8":
        n = moe_ffn.workspace_bytes_mxfp8(w.T, w.d, w.d_ff, w.E, w.k)
    else:
        n = moe_ffn.workspace_bytes(w.T, w.d, w.d_ff, w.E, w.k, dt, w.d_ff_shared, block=blk,
                                    grouped=w.routing == "grouped")
    return moe_ffn.alloc_workspace(n, device)


def run(w: Workload, t: dict, out=None, workspace=None, routing=False, stream=None,
        e_score_bias=None):
    """One layer (or block) forward of workload `w` on device tensors `t`."""
    block = block_of(w, t)
    if w.weights in ("affine4", "affine8"):
        return moe_ffn.forward_grouped_affine(
            moe_ffn.make_affine(4 if w.weights == "affine4" else 8, t), t["x"], t["router_w"], t.get("router_b"),
            w.k, w.n_group, w.topk_group, w.norm_topk_prob, w.routed_scaling_factor, w.d_ff,
            score=moe_ffn.MOE_SCORE_SOFTMAX if w.score == "softmax" else moe_ffn.MOE_SCORE_SIGMOID,
            act=moe_ffn.MOE_ACT_SILU if w.act == "silu" else moe_ffn.MOE_ACT_CLIPPED_SWIGLU,
            alpha=w.alpha, limit=w.limit, e_score_bias=e_score_bias, b_gate=t.get("b_gate"), b_up=t.get("b_up"),
            b_down=t.get("b_down"), shared_w_gate=t.get("shared_w_gate"), shared_w_up=t.get("shared_w_up"),
            shared_w_down=t.get("shared_w_down"), E=w.E, out=out, workspace=workspace, routing=routing,
            stream=stream, block=block)
    if w.routing == "grouped":
        return moe_ffn.forward_grouped(
            t["x"], t["router_w"], t.get("router_b"), t.get("w_gate"), t.get("b_gate"), t.get("w_up"),
            t.get("b_up"), t.get("w_down"), t.get("b_down"), w.k, w.n_group, w.topk_group,
            w.norm_topk_prob, w.routed_scaling_factor,
            score=moe_ffn.MOE_SCORE_SOFTMAX if w.score == "softmax" else moe_ffn.MOE_SCORE_SIGMOID,
            act=moe_ffn.MOE_ACT_SILU if w.act == "silu" else moe_ffn.MOE_ACT_CLIPPED_SWIGLU,
            alpha=w.alpha, limit=w.limit, e_score_bias=e_score_bias,
            shared_w_gate=t.get("shared_w_gate"), shared_w_up=t.get("shared_w_up"),
            shared_w_down=t.get("shared_w_down"), out=out, workspace=workspace, routing=routing,
            stream=stream, block=block)
    if w.act_quant == "mxfp8":
        if w.weights not in ("mxfp4", "mxfp8") or w.block:
            raise ValueError("MXFP8 activations are implemented for the plain MXFP4 / MXFP8 layer")
        return moe_ffn.forward_mxfp4_mxfp8(
            t["x"], t["router_w"], t.get("router_b"), t["w_gate_codes"], t["w_gate_scales"], t.get("b_gate"),
            t["w_up_codes"], t["w_up_scales"], t.get("b_up"), t["w_down_codes"], t["w_down_scales"],
            t.get("b_down"), w.k, alpha=w.alpha, limit=w.limit, out=out, workspace=workspace,
            routing=routing, stream=stream, weights=w.weights)
    if w.weights == "nvfp4":
        return moe_ffn.forward_nvfp4(
            t["x"], t["router_w"], t.get("router_b"), t["w_gate_codes"], t["w_gate_scales"],
            float(t["w_gate_tensor_scale"]), t.get("b_gate"), t["w_up_codes"], t["w_up_scales"],
            float(t["w_up_tensor_scale"]), t.get("b_up"), t["w_down_codes"], t["w_down_scales"],
            float(t["w_down_tensor_scale"]), t.get("b_down"), w.k, alpha=w.alpha, limit=w.limit, out=out,
            workspace=workspace, routing=routing, stream=stream)
    if w.weights == "mxfp4":
        return moe_ffn.forward_mxfp4(
            t["x"], t["router_w"], t.get("router_b"), t["w_gate_codes"], t["w_gate_scales"], t.get("b_gate"),
            t["w_up_codes"], t["w_up_scales"], t.get("b_up"), t["w_down_codes"], t["w_down_scales"],
            t.get("b_down"), w.k, alpha=w.alpha, limit=w.limit, out=out, workspace=workspace,
            routing=routing, stream=stream, block=block)
    return moe_ffn.forward(
        t["x"], t["router_w"], t.get("router_b"), t["w_gate"], t.get("b_gate"), t["w_up"], t.get("b_up"),
        t["w_down"], t.get("b_down"), w.k, alpha=w.alpha, limit=w.limit, out=out, workspace=workspace,
        routing=routing, stream=stream, block=block)
