"""Comparison of the GPU layer against the float64 oracle (test infrastructure).

Rules (same on every workload):
  * routing indices: bit-exact, in order, for every token whose routing margin
    (gap at the top-k boundary, and at the group boundary for grouped
    routing) is at least 1e-5 in logit space; tokens whose chosen experts
    are separated by less than 1e-5 among themselves are compared as sets;
    tokens below the boundary margin must make a valid choice within 1e-5
    and are checked on their outputs with the oracle forced to that choice;
  * routing weights: within 1e-5 absolute (fp32 router);
  * permutation: expert offsets and sorted pairs re-derived by the oracle
    from the GPU's own indices, bit-exact;
  * outputs: max |gpu - ref| <= tol * max |ref| over the checked tokens, with
    tol = 1e-4 for fp32 layers and 2e-2 for bf16 / MXFP4 / MXFP8-activation
    layers; every output element must have been written (the output is
    pre-filled with NaN);
  * MXFP8 activations: x converts exactly on both sides (it is bf16), but the
    E4M3 code of an element of h is a decision taken on a value that the GPU
    accumulates in fp32 and the oracle in fp64.  Where the oracle's g or u
    moved by the GPU's accumulation error (H_REL of the sum of the products'
    magnitudes) would change an element's code, either code is correct; each
    output's bound grows by what those alternatives can change it (the
    largest code change times |W_down| and the routing weight), as the
    routing near-ties are compared on what is unique.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import moe_oracle as O

MARGIN = 1e-5
# Relative accumulation error of g and u on the GPU (fp32 sums of MFMA
# results that are themselves exact to ~1.2e-4 of the block's sum of product
# magnitudes), as a fraction of the sum of |products|; used for the h codes.
H_REL = 3e-4


def cfg_of(w, e_score_bias=None) -> dict:
    c = dict(dtype=w.dtype, weights=w.weights, routing=w.routing, act=w.act, alpha=w.alpha,
             limit=w.limit, k=w.k, E=w.E, n_group=w.n_group, topk_group=w.topk_group,
             norm_topk_prob=w.norm_topk_prob, routed_scaling_factor=w.routed_scaling_factor,
             score=w.score, block=w.block, norm_eps=w.norm_eps, act_quant=w.act_quant)
    if e_score_bias is not None:
        c["e_score_bias"] = np.asarray(e_score_bias, dtype=np.float64)
    return c


def tolerance(w) -> float:
    return 1e-4 if w.dtype == "f32" else 2e-2


def sample_tokens(T: int, n_max: int, seed: int = 0) -> np.ndarray:
    """All tokens when T <= n_max; else the first and last 32 tokens plus a seeded sample."""
    if T <= n_max:
        return np.arange(T)
    rng = np.random.default_rng(seed)
    ends = np.concatenate([np.arange(32), np.arange(T - 32, T)])
    mid = rng.choice(np.arange(32, T - 32), size=n_max - 64, replace=False)
    return np.unique(np.concatenate([ends, mid]))


def check_layer(w, a: dict, gpu_out: torch.Tensor, r: dict, n_out_tokens: int = 512,
                e_score_bias=None) -> dict:
    """Compare one GPU forward (output + routing tensors) with the oracle.
    Returns a small report; raises AssertionError on any mismatch."""
    cfg = cfg_of(w, e_score_bias)
    T, k, E = w.T, w.k, w.E
    out = gpu_out.float().cpu().numpy().astype(np.float64)
    assert not np.isnan(out).any(), "output element not written (NaN sentinel survived) or NaN produced"
    g_idx = r["topk_idx"].cpu().numpy().astype(np.int64)
    g_w = r["topk_w"].cpu().numpy().astype(np.float64)
    g_off = r["expert_offsets"].cpu().numpy().astype(np.int64)
    g_sp = r["sorted_pair"].cpu().numpy().astype(np.int64)

    logits, o_idx, o_w = O.route(a, cfg)
    boundary, inner = O.route_margins(logits, cfg)
    clear = boundary >= MARGIN
    ordered = clear & (inner >= MARGIN)

    # indices
    bad = np.nonzero(ordered & np.any(g_idx != o_idx, axis=1))[0]
    assert bad.size == 0, f"routing differs on {bad.size} tokens, e.g. t={bad[:5]}: gpu {g_idx[bad[:3]]} oracle {o_idx[bad[:3]]}"
    sets_only = clear & ~ordered
    for t in np.nonzero(sets_only)[0]:
        assert set(g_idx[t]) == set(o_idx[t]), f"token {t}: expert sets differ"
    near = np.nonzero(~clear)[0]
    for t in near:
        gl = logits[t, g_idx[t]]
        ol = logits[t, o_idx[t]]
        assert len(set(g_idx[t])) == k and gl.min() >= ol.min() - MARGIN, f"token {t}: invalid near-tie choice"

    # weights (oracle weights of the GPU's choice, matched per expert)
    fw = O.forced_weights(logits, g_idx, cfg)
    np.testing.assert_allclose(g_w, fw, rtol=0, atol=1e-5 * max(1.0, float(np.abs(fw).max())))

    # permutation, re-derived from the GPU's own indices
    counts, offsets, sp, pos = O.permutation(g_idx, E)
    np.testing.assert_array_equal(g_off, offsets)
    np.testing.assert_array_equal(g_sp, sp)

    # outputs on the checked tokens
    toks = sample_tokens(T, n_out_tokens)
    use_gpu_choice = ~clear[toks] | sets_only[toks]
    idx_mix = np.where(use_gpu_choice[:, None], g_idx[toks], o_idx[toks])
    w_mix = np.where(use_gpu_choice[:, None], fw[toks], o_w[toks])
    ref = O.experts_forward(a, cfg, idx_mix, w_mix, tokens=toks)
    scale = np.abs(ref).max()
    tol = tolerance(w)
    extra = h_code_slack(a, cfg, idx_mix, w_mix, toks) if cfg.get("act_quant") == "mxfp8" else 0.0
    excess = np.abs(out[toks] - ref) - extra
    err = np.abs(out[toks] - ref).max()
    assert excess.max() <= tol * scale, (f"max|err| - slack = {excess.max():.3e} > {tol} * max|ref| = {tol * scale:.3e} "
                                         f"(max|err| {err:.3e})")
    return {"tokens_checked": int(toks.size), "near_ties": int(near.size), "set_ties": int(sets_only.sum()),
            "max_err": float(err), "max_ref": float(scale), "rel": float(err / scale),
            "rel_beyond_slack": float(excess.max() / scale),
            "max_slack_rel": float(np.max(extra) / scale) if np.ndim(extra) else 0.0}


def h_code_slack(a: dict, cfg: dict, idx: np.ndarray, wts: np.ndarray, toks: np.ndarray) -> np.ndarray:
    """Per output element, how far the output may move because E4M3 codes of h
    that sit within the accumulation error of a rounding decision can go
    either way (MXFP8-activation layers; see the module docstring)."""
    dt = cfg["dtype"]
    x = O.layer_input(a, cfg, toks)
    W = O.ExpertWeights(a, dt, cfg.get("weights", "dense"))
    alpha, limit = cfg.get("alpha", 1.702), cfg.get("limit", 7.0)
    slack = np.zeros((toks.size, x.shape[1]))
    for e in np.unique(idx):
        t_sel, j_sel = np.nonzero(idx == e)
        Wg, bg, Wu, bu, Wd, bd = W.expert(int(e))
        X = O.mxfp8_round(x[t_sel])
        g, u = X @ Wg.T, X @ Wu.T
        dg, du = H_REL * (np.abs(X) @ np.abs(Wg.T)), H_REL * (np.abs(X) @ np.abs(Wu.T))
        if bg is not None:
            g = g + bg
        if bu is not None:
            u = u + bu
        q0 = O.mxfp8_round(O.round_bf16(O.activation(g, u, "clipped_swiglu", alpha, limit)))
        dev = np.zeros_like(q0)
        for sg in (-1.0, 1.0):        # the activation is monotone in g and in u: corners bound it
            for su in (-1.0, 1.0):
                qc = O.mxfp8_round(O.round_bf16(O.activation(g + sg * dg, u + su * du, "clipped_swiglu", alpha, limit)))
                dev = np.maximum(dev, np.abs(qc - q0))
        slack[t_sel] += np.abs(wts[t_sel, j_sel])[:, None] * (dev @ np.abs(Wd.T))
    return slack
