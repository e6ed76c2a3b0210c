"""GPU parity of the HIP MoE-FFN layer against the float64 oracle, through the C ABI.

Each case prints its name, shape and seed before touching the GPU.
"""
import dataclasses
import sys

import numpy as np
import pytest
import torch

from mixture_experts_transformer_router_amd import inputs as I
from mixture_experts_transformer_router_amd import layer as LY
from mixture_experts_transformer_router_amd import moe_ffn
from mixture_experts_transformer_router_amd import workloads as W

from oracle import moe_oracle as O
from parity_util import cfg_of, check_layer

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def poisoned_workspace(w):
    """The layer's workspace filled with 0xFF bytes (NaN in bf16 and fp32, -1
    as int32): a kernel that reads a piece of it before writing it shows up
    as a NaN output or a wrong index."""
    return LY.workspace_for(w, DEV).fill_(0xFF)


def _run_and_check(w, a=None, n_out_tokens=512, e_score_bias=None):
    _say(f"[case] {w.name} T={w.T} d={w.d} F={w.d_ff} E={w.E} k={w.k} dtype={w.dtype} "
         f"weights={w.weights} routing={w.routing} score={w.score} seed={w.seed}")
    a = I.make_inputs(w) if a is None else a
    t = LY.to_device(a, DEV)
    out = torch.full((w.T, w.d), float("nan"), dtype=t["x"].dtype, device=DEV)
    eb = None if e_score_bias is None else torch.from_numpy(np.asarray(e_score_bias, np.float32)).to(DEV)
    ws = poisoned_workspace(w)
    out, r = LY.run(w, t, out=out, workspace=ws, routing=True, e_score_bias=eb)
    torch.cuda.synchronize()
    rep = check_layer(w, a, out, r, n_out_tokens=n_out_tokens, e_score_bias=e_score_bias, workspace=ws)
    _say(f"[ok] {w.name}: {rep}")
    return rep


# --- the five workloads at their full sizes ------------------------------------------

@pytest.mark.parametrize("w", W.ALL, ids=[w.name for w in W.ALL])
def test_workload_full_size(w):
    _run_and_check(w, n_out_tokens=256 if w.T > 256 else w.T)


# --- smaller shapes: several tiles, ragged tails, edge cases --------------------------

SMALL = [
    W.GPTOSS_DECODE.scaled(T=200, d=256, d_ff=192, E=8, k=2, name="gptoss_T200_ragged"),
    W.GPTOSS_DECODE.scaled(T=1, d=256, d_ff=128, E=32, k=4, name="gptoss_T1"),
    W.GPTOSS_DECODE.scaled(T=77, d=128, d_ff=64, E=1, k=1, name="dense_ffn_E1_k1"),
    W.GPTOSS_DECODE.scaled(T=65, d=64, d_ff=136, E=6, k=6, name="k_equals_E"),
    W.GPTOSS_DECODE.scaled(T=130, d=128, d_ff=64, E=256, k=16, name="E256_k16"),
    W.GPTOSS_PREFILL.scaled(T=1000, d=384, d_ff=320, name="prefill_zipf_small"),
    # grouped-GEMM path with K ragged against the 64-wide stages and many K
    # tiles (steady, unrolled and tail tiles): d = 1000, d_ff = 712
    W.GPTOSS_PREFILL.scaled(T=300, d=1000, d_ff=712, E=8, k=2, name="prefill_ragged_k"),
    # experts averaging two or more row tiles take the third weight stage:
    # steady, unrolled and tail K tiles; and K of one or two tiles (fewer
    # tiles than stages)
    W.GPTOSS_PREFILL.scaled(T=1100, d=1000, d_ff=712, E=4, k=2, name="prefill_deep_stages_ragged_k"),
    W.GPTOSS_PREFILL.scaled(T=1100, d=64, d_ff=96, E=4, k=2, name="prefill_deep_stages_short_k"),
    W.GPTOSS_MXFP4.scaled(T=150, d=256, d_ff=160, E=8, k=2, name="mxfp4_small"),
    W.TINY_F32.scaled(T=300, d=96, d_ff=80, E=16, k=3, name="f32_T300"),
    W.GLM4_MOE_LITE.scaled(T=300, d=256, d_ff=192, E=64, k=6, d_ff_shared=128, name="glm_small"),
    W.GLM4_MOE_LITE.scaled(T=120, d=128, d_ff=64, E=16, k=4, n_group=4, topk_group=2,
                           score="sigmoid", d_ff_shared=96, name="glm_sigmoid"),
    W.GLM4_MOE_LITE.scaled(T=90, d=64, d_ff=64, E=8, k=2, n_group=1, topk_group=1,
                           norm_topk_prob=False, routed_scaling_factor=2.5, d_ff_shared=0,
                           name="glm_no_shared_no_norm"),
    W.GLM4_MOE_LITE.scaled(T=70, d=96, d_ff=64, E=16, k=3, n_group=4, topk_group=2,
                           dtype="f32", act="clipped_swiglu", expert_bias=True, router_bias="normal",
                           d_ff_shared=32, name="glm_f32_clipped_shared"),
    # the shared expert beside the router and the permutation: one router
    # block pair and one row tile (T = 17), a shared expert wider than the
    # routed ones (its column tiles past the routed width), and more routed
    # experts than that path takes (E = 160: the shared tiles follow the
    # routed ones)
    W.GLM4_MOE_LITE.scaled(T=17, d=128, d_ff=64, E=16, k=4, n_group=4, topk_group=2, d_ff_shared=64,
                           name="glm_T17_shared"),
    W.GLM4_MOE_LITE.scaled(T=40, d=192, d_ff=64, E=16, k=4, n_group=4, topk_group=2, d_ff_shared=320,
                           name="glm_T40_wide_shared"),
    W.GLM4_MOE_LITE.scaled(T=100, d=128, d_ff=64, E=160, k=6, d_ff_shared=64, name="glm_E160_shared"),
    # few-token (weight-streaming) path: K ragged against 512-element chunks,
    # weight rows ragged against the 16-row blocks, 1 .. 16 rows per expert
    W.GPTOSS_DECODE.scaled(T=5, d=520, d_ff=72, E=8, k=3, name="decode_T5_ragged"),
    W.GPTOSS_DECODE.scaled(T=16, d=1096, d_ff=200, E=4, k=4, name="decode_T16_every_expert_full"),
    W.GPTOSS_DECODE.scaled(T=11, d=64, d_ff=24, E=3, k=2, name="decode_T11_short_rows"),
    W.GLM4_MOE_LITE.scaled(T=12, d=576, d_ff=96, E=16, k=4, n_group=4, topk_group=2,
                           d_ff_shared=160, name="glm_decode_T12_shared"),
    W.GLM4_MOE_LITE.scaled(T=3, d=1024, d_ff=256, E=64, k=6, d_ff_shared=40, name="glm_decode_T3"),
    # rows of 257 16-byte vectors: the combine's second block per token holds one
    W.GPTOSS_DECODE.scaled(T=3, d=2056, d_ff=64, E=4, k=2, name="decode_T3_d2056"),
    W.GPTOSS_PREFILL.scaled(T=40, d=2056, d_ff=96, E=4, k=2, name="prefill_T40_d2056"),
]


@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
def test_small_shapes(w):
    _run_and_check(w)


# The gate of the GLM page's MoEGate.Forward: sigmoid scores, a correction bias
# for the selection, no group limit (n_group = topk_group = 1).
PAGES_GATE = W.GLM4_MOE_LITE.scaled(n_group=1, topk_group=1, score="sigmoid",
                                    name="glm4moelite_pages_gate_sigmoid_ebias_T2048")


def _ebias(w, seed=7, std=0.05):
    return np.random.default_rng(seed).normal(0, std, w.E)


@pytest.mark.parametrize("w", [PAGES_GATE, PAGES_GATE.scaled(T=300, d=256, d_ff=192, d_ff_shared=128,
                                                              name="pages_gate_small"),
                               PAGES_GATE.scaled(T=12, d=576, d_ff=96, E=16, k=4, d_ff_shared=160,
                                                 name="pages_gate_decode_T12")],
                         ids=lambda w: w.name)
def test_pages_gate_sigmoid_with_correction_bias(w):
    _run_and_check(w, n_out_tokens=256 if w.T > 256 else w.T, e_score_bias=_ebias(w))


def test_grouped_sigmoid_full_size():
    w = W.GLM4_MOE_LITE.scaled(score="sigmoid", name="glm4moelite_sigmoid_T2048")
    _run_and_check(w, n_out_tokens=256)


def test_grouped_sigmoid_with_bias_and_groups_full_size():
    w = W.GLM4_MOE_LITE.scaled(score="sigmoid", name="glm4moelite_sigmoid_ebias_groups_T2048")
    _run_and_check(w, n_out_tokens=256, e_score_bias=_ebias(w, seed=8))


def test_grouped_with_correction_bias():
    w = W.GLM4_MOE_LITE.scaled(T=100, d=128, d_ff=64, E=32, k=4, n_group=8, topk_group=3,
                               d_ff_shared=64, name="glm_ebias")
    eb = np.random.default_rng(5).normal(0, 0.01, w.E)
    _run_and_check(w, e_score_bias=eb)


def test_all_tokens_on_one_expert():
    w = W.GPTOSS_DECODE.scaled(T=300, d=128, d_ff=64, E=8, k=1, name="one_expert")
    a = I.make_inputs(w)
    b = np.zeros(w.E, np.float32)
    b[5] = 1000.0
    a["router_b"] = I.f32_to_bf16_bits(b)
    rep = _run_and_check(w, a=a)
    assert rep["tokens_checked"] == 300


def test_mxfp4_nan_scale_gives_nan_exactly_where_the_block_is_used():
    # e8m0 byte 255 is NaN (OCP MX v1.0): a NaN gate block makes every output
    # of the tokens routed to that expert NaN; a NaN down block only the one
    # output column of those tokens.  Everything else must stay finite and
    # match the oracle under the GPU's own routing.
    w = W.GPTOSS_MXFP4.scaled(T=150, d=256, d_ff=160, E=8, k=2, name="mxfp4_nan_scale")
    a = I.make_inputs(w)
    a["w_gate_scales"] = a["w_gate_scales"].copy()
    a["w_gate_scales"][3, 5, 1] = 255     # expert 3, gate row 5, elements 32..63
    a["w_down_scales"] = a["w_down_scales"].copy()
    a["w_down_scales"][6, 10, 4] = 255    # expert 6, output column 10, elements 128..159
    _say(f"[case] {w.name} T={w.T} d={w.d} F={w.d_ff} E={w.E} k={w.k} seed={w.seed}")
    t = LY.to_device(a, DEV)
    out = torch.full((w.T, w.d), 3.0, dtype=torch.bfloat16, device=DEV)
    out, r = LY.run(w, t, out=out, routing=True)
    torch.cuda.synchronize()
    cfg = cfg_of(w)
    g_idx = r["topk_idx"].cpu().numpy().astype(np.int64)
    logits, _, _ = O.route(a, cfg)
    ref = O.experts_forward(a, cfg, g_idx, O.forced_weights(logits, g_idx, cfg))
    got = out.float().cpu().numpy().astype(np.float64)
    nan_ref = np.isnan(ref)
    rows_all_nan = nan_ref.all(axis=1)
    assert rows_all_nan.any(), "no token routed to expert 3"
    assert (nan_ref[~rows_all_nan, 10]).any(), "no token routed to expert 6 alone"
    np.testing.assert_array_equal(np.isnan(got), nan_ref)
    fin = ~nan_ref
    err = np.abs(got[fin] - ref[fin]).max()
    assert err <= 2e-2 * np.abs(ref[fin]).max(), err
    _say(f"[ok] {w.name}: nan rows {int(rows_all_nan.sum())}, max err {err:.3e}")


def test_exact_logit_ties_lowest_index_wins():
    # identical router rows => identical logits for experts 0..3: ties go to 0, 1
    w = W.GPTOSS_DECODE.scaled(T=64, d=64, d_ff=64, E=4, k=2, name="exact_ties")
    a = I.make_inputs(w)
    a["router_w"][:] = a["router_w"][0:1]
    t = LY.to_device(a, DEV)
    _say("[case] exact_ties")
    out, r = LY.run(w, t, routing=True)
    torch.cuda.synchronize()
    idx = r["topk_idx"].cpu().numpy()
    np.testing.assert_array_equal(idx, np.tile([[0, 1]], (w.T, 1)))
    np.testing.assert_allclose(r["topk_w"].cpu().numpy(), 0.5)


def test_deterministic_and_token_permutation_equivariant():
    w = W.GPTOSS_PREFILL.scaled(T=700, d=256, d_ff=192, E=16, k=4, name="determinism")
    _say(f"[case] {w.name}")
    a = I.make_inputs(w)
    t = LY.to_device(a, DEV)
    o1 = LY.run(w, t)
    o2 = LY.run(w, t)
    perm = np.random.default_rng(3).permutation(w.T)
    a2 = dict(a)
    a2["x"] = a["x"][perm]
    t2 = LY.to_device(a2, DEV)
    o3 = LY.run(w, t2)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(o1[torch.from_numpy(perm).to(DEV)].view(torch.int16), o3.view(torch.int16))


DETERMINISM = [
    W.GPTOSS_DECODE,                        # weight-streaming kernels (bf16)
    W.GPTOSS_MXFP4_DECODE,                  # weight-streaming kernels on MXFP4 codes
    W.GPTOSS_MXFP4.scaled(T=600, name="mxfp4_T600"),          # low-bit GEMM (MXFP4)
    W.GPTOSS_MXFP4_MX8.scaled(T=600, name="mxfp4_mx8_T600"),  # scaled MFMA
    W.GPTOSS_NVFP4.scaled(T=300, name="nvfp4_T300"),
    W.GLM4_MOE_LITE_INT4.scaled(T=600, name="int4_T600"),     # affine GEMM + bf16 shared expert
    W.GLM4_MOE_LITE.scaled(T=600, name="glm_T600"),
]


@pytest.mark.parametrize("w", DETERMINISM, ids=lambda w: w.name)
def test_repeat_calls_are_bitwise_identical(w):
    # every path sums in a fixed order: the same call twice gives the same bits
    _say(f"[case] determinism {w.name} T={w.T}")
    t = LY.to_device(I.make_inputs(w), DEV)
    o1 = LY.run(w, t, workspace=poisoned_workspace(w))
    o2 = LY.run(w, t, workspace=poisoned_workspace(w))
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


@pytest.mark.parametrize("base", [W.GLM4_MOE_LITE, W.GLM4_MOE_LITE_INT4], ids=["bf16", "int4"])
def test_interleaved_calls_on_two_caller_streams(base):
    # Calls on two caller streams, each with its own workspace, queued
    # alternately with no synchronisation: every call must match the oracle
    # (the library keeps no state between calls and enqueues only on the
    # stream it is given), and a repeat of the first call on the other stream
    # must give the same bits.
    w1 = base.scaled(T=600, d=256, d_ff=192, E=64, k=6, d_ff_shared=192, name=f"two_streams_{base.weights}")
    w2 = w1.scaled(seed=w1.seed + 1)
    _say(f"[case] {w1.name} T={w1.T} two streams")
    a1, a2 = I.make_inputs(w1), I.make_inputs(w2)
    t1, t2 = LY.to_device(a1, DEV), LY.to_device(a2, DEV)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    ws1, ws2 = poisoned_workspace(w1), poisoned_workspace(w2)
    outs = [torch.full((w1.T, w1.d), float("nan"), dtype=torch.bfloat16, device=DEV) for _ in range(4)]
    torch.cuda.synchronize()
    o1, r1 = LY.run(w1, t1, out=outs[0], workspace=ws1, routing=True, stream=s1)
    o2, r2 = LY.run(w2, t2, out=outs[1], workspace=ws2, routing=True, stream=s2)
    o3 = LY.run(w1, t1, out=outs[2], workspace=ws1, stream=s1)
    o4 = LY.run(w1, t1, out=outs[3], workspace=ws2, stream=s2)   # after o2 on s2: its workspace is free
    torch.cuda.synchronize()
    check_layer(w1, a1, o1, r1, n_out_tokens=128)
    check_layer(w2, a2, o2, r2, n_out_tokens=128)
    assert torch.equal(o1.view(torch.int16), o3.view(torch.int16))
    assert torch.equal(o1.view(torch.int16), o4.view(torch.int16))


def test_zero_tokens_is_noop_and_errors_leave_out_untouched():
    w = W.GPTOSS_DECODE.scaled(T=16, d=64, d_ff=64, E=4, k=2, name="errors")
    _say("[case] errors")
    t = LY.to_device(I.make_inputs(w), DEV)
    out = torch.full((w.T, w.d), 3.0, dtype=torch.bfloat16, device=DEV)
    ws = LY.workspace_for(w, DEV)
    with pytest.raises(moe_ffn.MoeError) as ei:
        moe_ffn.forward(t["x"], t["router_w"], t["router_b"], t["w_gate"], t["b_gate"], t["w_up"],
                        t["b_up"], t["w_down"], t["b_down"], k=5, out=out, workspace=ws)
    assert ei.value.status == moe_ffn.MOE_ERR_INVALID_ARG
    small_ws = torch.empty(256, dtype=torch.uint8, device=DEV)
    with pytest.raises(moe_ffn.MoeError) as ei:
        moe_ffn.forward(t["x"], t["router_w"], t["router_b"], t["w_gate"], t["b_gate"], t["w_up"],
                        t["b_up"], t["w_down"], t["b_down"], k=2, out=out, workspace=small_ws)
    assert ei.value.status == moe_ffn.MOE_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)
    empty = moe_ffn.forward(t["x"][:0], t["router_w"], t["router_b"], t["w_gate"], t["b_gate"], t["w_up"],
                            t["b_up"], t["w_down"], t["b_down"], k=2)
    assert empty.shape == (0, w.d)

# --- MoE blocks: RMSNorm in front of the layer, residual after it -------------------

BLOCK_SMALL = [
    # every expert path: weight streaming (T <= 16), bf16 MFMA with ragged K,
    # MXFP4, fp32, grouped routing with a shared expert
    W.GPTOSS_DECODE.scaled(T=7, d=520, d_ff=72, E=8, k=3, block=True, name="block_decode_T7"),
    W.GPTOSS_PREFILL.scaled(T=300, d=1000, d_ff=712, E=8, k=2, block=True, name="block_prefill_ragged_k"),
    W.GPTOSS_MXFP4.scaled(T=150, d=256, d_ff=160, E=8, k=2, block=True, name="block_mxfp4_small"),
    W.TINY_F32.scaled(T=40, d=96, d_ff=80, E=16, k=3, block=True, name="block_f32"),
    W.GLM4_MOE_LITE.scaled(T=300, d=256, d_ff=192, E=64, k=6, d_ff_shared=128, block=True,
                           name="block_glm_small"),
    W.GLM4_DENSE_BLOCK.scaled(T=100, d=256, d_ff=520, name="dense_block_small"),
    W.GLM4_DENSE_BLOCK.scaled(T=9, d=256, d_ff=136, name="dense_block_T9"),
    # rows longer than the norm kernel keeps in registers (two passes over x)
    W.GPTOSS_DECODE.scaled(T=4, d=16400, d_ff=16, E=4, k=2, block=True, name="block_bf16_d16400"),
    W.TINY_F32.scaled(T=6, d=8200, d_ff=16, E=4, k=2, block=True, name="block_f32_d8200"),
]
BLOCK_CASES = list(W.BLOCKS) + BLOCK_SMALL


@pytest.mark.parametrize("w", BLOCK_CASES, ids=[w.name for w in BLOCK_CASES])
def test_block(w):
    _run_and_check(w, n_out_tokens=256 if w.T > 256 else w.T)


def test_block_residual_only_and_norm_only():
    # residual without a norm = the plain layer plus x; a norm without the
    # residual = the full block minus x (each up to the roundings of the two
    # ways of computing it)
    w = W.GLM4_MOE_LITE.scaled(T=200, d=256, d_ff=192, E=16, k=4, n_group=4, topk_group=2, d_ff_shared=64,
                               block=True, name="block_parts")
    _say(f"[case] {w.name}")
    a = I.make_inputs(w)
    t = LY.to_device(a, DEV)
    plain = LY.run(dataclasses.replace(w, block=False), t)
    full = LY.run(w, t)
    x = t["x"].float()

    def grouped(block):
        return moe_ffn.forward_grouped(
            t["x"], t["router_w"], None, t["w_gate"], None, t["w_up"], None, t["w_down"], None, w.k, w.n_group,
            w.topk_group, w.norm_topk_prob, w.routed_scaling_factor, act=moe_ffn.MOE_ACT_SILU,
            shared_w_gate=t["shared_w_gate"], shared_w_up=t["shared_w_up"], shared_w_down=t["shared_w_down"],
            block=block)
    res_only = grouped(moe_ffn.make_block(None, 0.0, True))
    norm_only = grouped(moe_ffn.make_block(t["norm_w"], w.norm_eps, False))
    torch.cuda.synchronize()
    scale = float((x + plain.float()).abs().max())
    assert float((res_only.float() - (x + plain.float())).abs().max()) <= 2 ** -7 * scale
    scale = float(full.float().abs().max())
    assert float((norm_only.float() - (full.float() - x)).abs().max()) <= 2 ** -7 * scale
    assert float((norm_only.float() - plain.float()).abs().max()) > 1e-2  # the norm changes the layer


# --- affine group-quantized routed experts (INT4 groups of 32, INT8 groups of 64) ----

AFFINE_SMALL = [
    W.GLM4_MOE_LITE_INT4.scaled(T=300, d=256, d_ff=192, E=64, k=6, d_ff_shared=128, name="int4_small"),
    W.GLM4_MOE_LITE_INT8.scaled(T=300, d=256, d_ff=192, E=64, k=6, d_ff_shared=128, name="int8_small"),
    # K = 160 / 96: not a multiple of 64, the general kernel with a K tail
    W.GLM4_MOE_LITE_INT4.scaled(T=200, d=160, d_ff=96, E=16, k=4, n_group=4, topk_group=2, d_ff_shared=0,
                                name="int4_ragged_k_no_shared"),
    W.GLM4_MOE_LITE_INT8.scaled(T=5, d=512, d_ff=128, E=16, k=4, n_group=4, topk_group=2, d_ff_shared=64,
                                name="int8_T5"),
    W.GLM4_MOE_LITE_INT4.scaled(T=150, d=256, d_ff=128, E=16, k=4, n_group=4, topk_group=2, d_ff_shared=64,
                                block=True, name="int4_block"),
]
AFFINE_CASES = list(W.QUANTIZED) + AFFINE_SMALL


@pytest.mark.parametrize("w", AFFINE_CASES, ids=[w.name for w in AFFINE_CASES])
def test_affine_experts(w):
    _run_and_check(w, n_out_tokens=256 if w.T > 256 else w.T)



# --- MXFP4 weights x MXFP8 activations on the scaled MFMA -----------------------------

MX_CASES = [
    W.GPTOSS_MXFP4_MX8,
    # K in 128-wide stages: d = 256 two stages, d_ff = 192 one and a half
    W.GPTOSS_MXFP4_MX8.scaled(T=150, d=256, d_ff=192, E=8, k=2, name="mx8_small"),
    # one token; gate|up one whole stage, down one half stage
    W.GPTOSS_MXFP4_MX8.scaled(T=1, d=128, d_ff=64, E=32, k=4, name="mx8_T1"),
    # several row tiles per expert, 4.5 / 3.5 stages (steady pairs, then the tail)
    W.GPTOSS_MXFP4_MX8.scaled(T=600, d=576, d_ff=448, E=4, k=2, name="mx8_many_tiles"),
    # k = E; gate|up a single half stage
    W.GPTOSS_MXFP4_MX8.scaled(T=70, d=64, d_ff=320, E=6, k=6, name="mx8_k_equals_E"),
    # few tokens, long K (8 stages), N ragged against the 256-column tiles
    W.GPTOSS_MXFP4_MX8.scaled(T=9, d=1024, d_ff=320, E=8, k=3, name="mx8_T9_long_k"),
    # long K: gate|up 25 stages, down 16.5 (a half stage after 8 steady pairs)
    W.GPTOSS_MXFP4_MX8.scaled(T=40, d=3200, d_ff=2112, E=4, k=2, name="mx8_long_k_d3200"),
    # MXFP8 (E4M3) weights: the full layer, 1.5 / 4.5 stages, a single half stage
    W.GPTOSS_MXFP8_MX8,
    W.GPTOSS_MXFP8_MX8.scaled(T=150, d=256, d_ff=192, E=8, k=2, name="mx8w_small"),
    W.GPTOSS_MXFP8_MX8.scaled(T=600, d=576, d_ff=448, E=4, k=2, name="mx8w_many_tiles"),
    W.GPTOSS_MXFP8_MX8.scaled(T=70, d=64, d_ff=320, E=6, k=6, name="mx8w_k_equals_E"),
]


@pytest.mark.parametrize("w", MX_CASES, ids=[w.name for w in MX_CASES])
def test_mxfp8_activation_layer(w):
    _run_and_check(w, n_out_tokens=256 if w.T > 256 else w.T)


def test_mxfp8_quantize_matches_oracle_bit_exactly():
    # the activation step alone: every code and scale byte must equal the oracle's
    rng = np.random.default_rng(11)
    rows, cols = 96, 320
    v = rng.standard_normal((rows, cols)) * np.ldexp(1.0, rng.integers(-40, 40, (rows, 1)))
    v[0, :32] = 0.0
    v[1, 32:64] = -0.0
    v[2, :32] = np.ldexp(rng.integers(-7, 8, 32).astype(np.float64), -133)   # bf16 subnormals
    v[3, :] = rng.standard_normal(cols) * 1e37                                 # near the top of bf16
    # exact E4M3 ties after scaling (max 1.0 -> scale 2^-8): 17/256, 19/256, and subnormal ties
    v[4, :32] = 0.0
    v[4, 0], v[4, 1], v[4, 2], v[4, 3], v[4, 4] = 1.0, 17 / 256, -19 / 256, 3 * 2.0 ** -18, 2.0 ** -18
    v[5, :32] = 1.8125                                                          # saturation at 448
    bits = I.f32_to_bf16_bits(v.astype(np.float32))
    bits[6, 5] = 0x7FC0       # NaN
    bits[7, 40] = 0x7F80      # +inf
    bits[8, 70] = 0xFF80      # -inf
    _say(f"[case] mxfp8_quantize rows={rows} cols={cols} seed=11")
    x = LY.to_device({"x": bits}, DEV)["x"]
    codes, scales = moe_ffn.mxfp8_quantize(x)
    torch.cuda.synchronize()
    ref_c, ref_s = O.mxfp8_quantize(O.bf16_to_f64(bits))
    np.testing.assert_array_equal(scales.cpu().numpy(), ref_s)
    np.testing.assert_array_equal(codes.cpu().numpy(), ref_c)
    assert ref_s[6, 0] == 255 and ref_s[7, 1] == 255 and ref_s[8, 2] == 255 and ref_s[0, 0] == 0


def test_mxfp8_activation_nan_scale():
    # a NaN weight scale: the gate block's NaN reaches h, whose MXFP8 block then
    # takes the NaN scale, so every output of those tokens is NaN; a NaN down
    # block makes one output column NaN.  Elsewhere the oracle's values.
    w = W.GPTOSS_MXFP4_MX8.scaled(T=150, d=256, d_ff=192, E=8, k=2, name="mx8_nan_scale")
    a = I.make_inputs(w)
    a["w_gate_scales"] = a["w_gate_scales"].copy()
    a["w_gate_scales"][3, 5, 1] = 255
    a["w_down_scales"] = a["w_down_scales"].copy()
    a["w_down_scales"][6, 10, 4] = 255
    _say(f"[case] {w.name} T={w.T} d={w.d} F={w.d_ff} E={w.E} k={w.k} seed={w.seed}")
    t = LY.to_device(a, DEV)
    out = torch.full((w.T, w.d), 3.0, dtype=torch.bfloat16, device=DEV)
    out, r = LY.run(w, t, out=out, routing=True)
    torch.cuda.synchronize()
    cfg = cfg_of(w)
    g_idx = r["topk_idx"].cpu().numpy().astype(np.int64)
    logits, _, _ = O.route(a, cfg)
    ref = O.experts_forward(a, cfg, g_idx, O.forced_weights(logits, g_idx, cfg))
    got = out.float().cpu().numpy().astype(np.float64)
    nan_ref = np.isnan(ref)
    assert nan_ref.all(axis=1).any() and nan_ref[~nan_ref.all(axis=1), 10].any()
    np.testing.assert_array_equal(np.isnan(got), nan_ref)
    fin = ~nan_ref
    assert np.abs(got[fin] - ref[fin]).max() <= 2e-2 * np.abs(ref[fin]).max()


# --- NVFP4 weights (e2m1, E4M3 scale per 16, tensor scale), decoded in registers --------

NV_CASES = [
    W.GPTOSS_NVFP4,
    W.GPTOSS_NVFP4.scaled(T=150, d=256, d_ff=192, E=8, k=2, name="nvfp4_small"),
    # K ragged against the 64-wide tiles: the general kernel (scales in registers, a K tail)
    W.GPTOSS_NVFP4.scaled(T=90, d=96, d_ff=160, E=6, k=3, name="nvfp4_ragged_k"),
    W.GPTOSS_NVFP4.scaled(T=1, d=128, d_ff=64, E=32, k=4, name="nvfp4_T1"),
]


@pytest.mark.parametrize("w", NV_CASES, ids=[w.name for w in NV_CASES])
def test_nvfp4_layer(w):
    _run_and_check(w, n_out_tokens=256 if w.T > 256 else w.T)


def test_nvfp4_nan_scale():
    # an E4M3 NaN scale (0x7F) in a gate block makes every output of the tokens
    # routed to that expert NaN; one in a down block only that output column
    w = W.GPTOSS_NVFP4.scaled(T=150, d=256, d_ff=192, E=8, k=2, name="nvfp4_nan_scale")
    a = I.make_inputs(w)
    a["w_gate_scales"] = a["w_gate_scales"].copy()
    a["w_gate_scales"][3, 5, 3] = 0x7F     # expert 3, gate row 5, elements 48..63
    a["w_down_scales"] = a["w_down_scales"].copy()
    a["w_down_scales"][6, 10, 9] = 0xFF    # expert 6, output column 10, elements 144..159
    _say(f"[case] {w.name} T={w.T} d={w.d} F={w.d_ff} E={w.E} k={w.k} seed={w.seed}")
    t = LY.to_device(a, DEV)
    out = torch.full((w.T, w.d), 3.0, dtype=torch.bfloat16, device=DEV)
    out, r = LY.run(w, t, out=out, routing=True)
    torch.cuda.synchronize()
    cfg = cfg_of(w)
    g_idx = r["topk_idx"].cpu().numpy().astype(np.int64)
    logits, _, _ = O.route(a, cfg)
    ref = O.experts_forward(a, cfg, g_idx, O.forced_weights(logits, g_idx, cfg))
    got = out.float().cpu().numpy().astype(np.float64)
    nan_ref = np.isnan(ref)
    assert nan_ref.all(axis=1).any() and nan_ref[~nan_ref.all(axis=1), 10].any()
    np.testing.assert_array_equal(np.isnan(got), nan_ref)
    fin = ~nan_ref
    assert np.abs(got[fin] - ref[fin]).max() <= 2e-2 * np.abs(ref[fin]).max()


# --- MXFP4 weights at decode (T <= 16): the weight-streaming kernel ---------------------

MXD_CASES = [
    W.GPTOSS_MXFP4_DECODE,
    # 16 rows per expert: eight passes of 2 tokens over the weights
    W.GPTOSS_MXFP4_DECODE.scaled(T=16, d=512, d_ff=256, E=4, k=4, name="mxfp4_decode_T16_multi_pass"),
    # 7 tokens over 2 experts: an odd row count ends on a half-filled pass of 2
    W.GPTOSS_MXFP4_DECODE.scaled(T=7, d=320, d_ff=224, E=2, k=1, name="mxfp4_decode_T7_two_experts"),
    # K = 2112 (66 blocks of 32): 32 lanes per row, the last of 3 steps with 2 lanes busy; 1..5 rows per expert
    W.GPTOSS_MXFP4_DECODE.scaled(T=5, d=2112, d_ff=160, E=6, k=3, name="mxfp4_decode_T5_ragged_k"),
    # gate|up rows of 2048 (64 lanes per row), down rows of 3072 (96 blocks: 32 lanes per row, two rows a step)
    W.GPTOSS_MXFP4_DECODE.scaled(T=6, d=2048, d_ff=3072, E=4, k=2, name="mxfp4_decode_lanes_64_32"),
    # the full-size rows (32 lanes per row) with ~7 rows per expert: four passes of 2 tokens
    W.GPTOSS_MXFP4_DECODE.scaled(T=9, E=4, k=3, name="mxfp4_decode_T9_E4"),
    W.GPTOSS_MXFP4_DECODE.scaled(T=1, d=256, d_ff=96, E=32, k=4, name="mxfp4_decode_T1"),
    # as a MoE block
    W.GPTOSS_MXFP4_DECODE.scaled(T=8, d=256, d_ff=192, E=8, k=2, block=True, name="mxfp4_decode_block"),
]


@pytest.mark.parametrize("w", MXD_CASES, ids=[w.name for w in MXD_CASES])
def test_mxfp4_decode(w):
    _run_and_check(w)


def test_mxfp4_decode_nan_scale():
    # NaN e8m0 scales on the weight-streaming path: as on the GEMM path
    w = W.GPTOSS_MXFP4_DECODE.scaled(T=12, d=256, d_ff=192, E=4, k=2, name="mxfp4_decode_nan_scale")
    a = I.make_inputs(w)
    a["w_gate_scales"] = a["w_gate_scales"].copy()
    a["w_gate_scales"][1, 7, 2] = 255
    a["w_down_scales"] = a["w_down_scales"].copy()
    a["w_down_scales"][2, 20, 3] = 255
    _say(f"[case] {w.name} T={w.T} d={w.d} F={w.d_ff} E={w.E} k={w.k} seed={w.seed}")
    t = LY.to_device(a, DEV)
    out = torch.full((w.T, w.d), 3.0, dtype=torch.bfloat16, device=DEV)
    out, r = LY.run(w, t, out=out, routing=True)
    torch.cuda.synchronize()
    cfg = cfg_of(w)
    g_idx = r["topk_idx"].cpu().numpy().astype(np.int64)
    logits, _, _ = O.route(a, cfg)
    ref = O.experts_forward(a, cfg, g_idx, O.forced_weights(logits, g_idx, cfg))
    got = out.float().cpu().numpy().astype(np.float64)
    nan_ref = np.isnan(ref)
    assert nan_ref.any()
    np.testing.assert_array_equal(np.isnan(got), nan_ref)
    fin = ~nan_ref
    assert np.abs(got[fin] - ref[fin]).max() <= 2e-2 * np.abs(ref[fin]).max()
