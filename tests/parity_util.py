"""Comparison of the GPU layer against the float64 oracle (test infrastructure).

Rules (same on every workload):
  * routing indices: bit-exact, in order, for every token whose routing margin
    (gap at the top-k boundary, and at the group boundary for grouped
    routing) is at least 1e-5 in the space where the choice is made (the
    logits, or the scores plus the correction bias); tokens whose chosen
    experts are separated by less than 1e-5 among themselves are compared
    as sets; tokens below the boundary margin must make a valid choice
    within 1e-5 (valid_choice, groups included) and are checked on their
    outputs with the oracle forced to that choice;
  * routing weights: within 1e-5 absolute (fp32 router);
  * permutation: expert offsets and sorted pairs re-derived by the oracle
    from the GPU's own indices, bit-exact;
  * outputs: max |gpu - ref| <= tol * max |ref| over the checked tokens, with
    tol = 1e-4 for fp32 layers and 2e-2 for bf16 / MXFP4 / MXFP8-activation
    layers; every output element must have been written (the output is
    pre-filled with NaN);
  * MXFP8 activations: x converts exactly on both sides (it is bf16), but the
    E4M3 code of an element of h is a decision taken on a value that the GPU
    accumulates in fp32 and the oracle in fp64, so near a rounding boundary
    two codes are correct.  The check reads the GPU's codes and scales of h
    from the workspace (moe_ffn_mxfp8_h_layout) and requires each one to be
    admissible: reachable from some value of g, u and h within a bound
    derived from the scaled MFMA's arithmetic (products truncated in groups of
    8, fp32 sums) and the fp32 roundings after it (h_admissible_interval).  The
    oracle then continues from the GPU's h (the down product and the
    combine), and the outputs must agree within the plain 2e-2.
"""
from __future__ import annotations

import itertools

import numpy as np
import torch

from oracle import moe_oracle as O

MARGIN = 1e-5


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


def valid_choice(v: np.ndarray, choice: np.ndarray, cfg: dict, margin: float) -> bool:
    """Whether `choice` (k expert indices, best first) is a correct routing of
    one token whose selection values are v (oracle.selection_values) when
    values closer than `margin` may compare either way:
      * k distinct experts, listed in descending order of v (within margin);
      * GPT-OSS routing: no unchosen expert exceeds the smallest chosen value
        by more than margin;
      * grouped routing: some set S of topk_group groups contains every chosen
        expert's group, no group outside S has a group score (largest v in the
        group) above the smallest group score in S by more than margin, and no
        unchosen expert of S's groups exceeds the smallest chosen value by more
        than margin."""
    choice = [int(e) for e in choice]
    k, E = len(choice), v.size
    if len(set(choice)) != k or min(choice) < 0 or max(choice) >= E:
        return False
    vc = v[choice]
    if np.any(vc[1:] > vc[:-1] + margin):
        return False
    vmin = vc.min()
    chosen = np.zeros(E, dtype=bool)
    chosen[choice] = True
    if cfg.get("routing", "gptoss") != "grouped":
        return not np.any(v[~chosen] > vmin + margin)
    ng, tg = cfg["n_group"], cfg["topk_group"]
    gs = E // ng
    G = v.reshape(ng, gs).max(axis=1)
    need = sorted({e // gs for e in choice})
    if len(need) > tg:
        return False
    # a group below the tg-th largest score by more than margin is beaten by
    # at least one excluded group of larger score, so S draws only from these
    g_tg = np.sort(G)[::-1][tg - 1]
    cand = [g for g in range(ng) if g not in need and G[g] >= g_tg - margin]
    for extra in itertools.combinations(cand, tg - len(need)):
        S = set(need) | set(extra)
        inside = np.zeros(ng, dtype=bool)
        inside[list(S)] = True
        if np.any(G[~inside] > G[inside].min() + margin):
            continue
        allowed = np.repeat(inside, gs)
        if not np.any(v[allowed & ~chosen] > vmin + margin):
            return True
    return False


def check_layer(w, a: dict, gpu_out: torch.Tensor, r: dict, n_out_tokens: int = 512,
                e_score_bias=None, workspace: torch.Tensor = None) -> dict:
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
    sel = O.selection_values(logits, cfg)
    for t in near:
        assert valid_choice(sel[t], g_idx[t], cfg, MARGIN), \
            f"token {t}: choice {g_idx[t]} is not a valid near-tie choice (oracle {o_idx[t]})"

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
    extra = {}
    if cfg.get("act_quant") == "mxfp8":
        assert workspace is not None, "an MXFP8-activation layer is checked with its workspace"
        ref, differ = mx_layer_reference(w, a, cfg, g_idx, g_sp, fw[toks], toks, workspace)
        extra["h_codes_not_oracles"] = differ
    else:
        ref = O.experts_forward(a, cfg, idx_mix, w_mix, tokens=toks)
    scale = np.abs(ref).max()
    tol = tolerance(w)
    err = np.abs(out[toks] - ref).max()
    assert err <= tol * scale, f"max|err| = {err:.3e} > {tol} * max|ref| = {tol * scale:.3e}"
    return {"tokens_checked": int(toks.size), "near_ties": int(near.size), "set_ties": int(sets_only.sum()),
            "max_err": float(err), "max_ref": float(scale), "rel": float(err / scale), **extra}


# Arithmetic of v_mfma_scale_f32_32x32x64_f8f6f4 with E4M3 activations and
# E4M3 or e2m1 weights, established with deterministic one-row probes of the
# instruction and confirmed on a layer (mx_dot_model reproduces the GPU's
# codes of h): the 64 products of an instruction are summed in groups of 8
# consecutive k; within a group each product is truncated toward zero to a
# multiple of 2^(M - 13), where M is the largest e(x) + e(w) of the group and
# e() the exponent of an element's code (its exponent field, read as the
# smallest normal exponent for subnormal codes and zero) plus its block
# scale; the group sums and the accumulator are added with fp32
# round-to-nearest.
MX_GROUP = 8
MX_ALIGN_BITS = 13
# smallest normal exponent of the code formats
E4M3_EMIN, E2M1_EMIN = -6, 0


def code_exponent_floor(scales: np.ndarray, K: int, emin: int) -> np.ndarray:
    """2^(emin + block scale exponent) for each element of rows with e8m0
    block scales [n, K/32]: the smallest 2^e() an element of the block can
    have."""
    return np.repeat(np.ldexp(1.0, scales.astype(np.int64) - 127 + emin), 32, axis=1)[:, :K]


def mx_dot_model(X, Wm, x_emin_floor, w_emin_floor):
    """The scaled MFMA's dot products of rows X [n, K] with rows Wm [F, K]
    (exact MXFP8 / MXFP4 values, float64) as modelled above; the floors are
    code_exponent_floor() of X and Wm.  Returns float64 [n, F] (fp32 values).
    Test infrastructure: used to check that the admissible bound covers the
    instruction's arithmetic."""
    n, K = X.shape
    ex = np.floor(np.log2(np.maximum(np.abs(X), x_emin_floor)))
    ew = np.floor(np.log2(np.maximum(np.abs(Wm), w_emin_floor)))
    acc = np.zeros((n, Wm.shape[0]), np.float32)
    for g0 in range(0, K, MX_GROUP):
        P = X[:, None, g0:g0 + MX_GROUP] * Wm[None, :, g0:g0 + MX_GROUP]
        M = (ex[:, None, g0:g0 + MX_GROUP] + ew[None, :, g0:g0 + MX_GROUP]).max(axis=2, keepdims=True)
        q = np.ldexp(1.0, (M - MX_ALIGN_BITS).astype(np.int32))
        acc = (acc + (np.trunc(P / q) * q).sum(axis=2).astype(np.float32)).astype(np.float32)
    return acc.astype(np.float64)


def h_admissible_interval(X, x_floor, Wg, wg_floor, bg, Wu, wu_floor, bu, alpha: float, limit: float):
    """Bounds on the fp32 value of h = clipped_swiglu(g, u) that the GPU
    computes for rows X (float64, the exact MXFP8 values of the token rows)
    of one expert; *_floor are code_exponent_floor() of X and of the weights.
    Returns (h, lo, hi) in float64.

    Derivation.  g = X Wg^T + bg (the same for u).  In each group of 8 the
    scaled MFMA loses less than 2^(M - 13) per product, with
    2^M <= max_g x~ * max_g w~, x~ = max(|x|, its floor) >= 2^e(x): in all
    below 8 * 2^-13 * sum_g max_g x~ max_g w~.  The K/8 group sums, the
    accumulator and the bias are then added in fp32 with round-to-nearest:
    at most K/8 + 2 roundings of partial sums no larger than
    S = sum |products| + |bias|, at most gamma_{K/8+2} S with
    gamma_n = n u / (1 - n u), u = 2^-24.  The clipped SwiGLU
    g' sigmoid(alpha g') u' is the product of two factors, each monotone in
    one argument, so over the box g +- dg, u +- du its extremes sit at the
    corners.  Its fp32 evaluation adds at most (2 alpha limit + 16) 2^-23 of
    |h|: the exponent's argument |z| <= alpha limit carries one rounding (an
    error |z| u of exp), the hardware exp2 and reciprocal one ulp each, and
    five more roundings (alpha g', 1 + e, the products)."""
    n, K = X.shape
    assert K % MX_GROUP == 0
    G = K // MX_GROUP
    nr = G + 2
    u = 2.0 ** -24
    gamma = nr * u / (1.0 - nr * u)
    Xt = np.maximum(np.abs(X), x_floor).reshape(n, G, MX_GROUP).max(axis=2)
    Xa = np.abs(X)

    def bound(Wm, w_floor, b):
        Wa = np.abs(Wm)
        Wt = np.maximum(Wa, w_floor).reshape(Wa.shape[0], G, MX_GROUP).max(axis=2)
        S = Xa @ Wa.T + (0.0 if b is None else np.abs(b))
        return MX_GROUP * 2.0 ** -MX_ALIGN_BITS * (Xt @ Wt.T) + gamma * S

    g, u_ = X @ Wg.T, X @ Wu.T
    if bg is not None:
        g = g + bg
    if bu is not None:
        u_ = u_ + bu
    dg, du = bound(Wg, wg_floor, bg), bound(Wu, wu_floor, bu)
    h = O.clipped_swiglu(g, u_, alpha, limit)
    corners = [O.clipped_swiglu(g + sg * dg, u_ + su * du, alpha, limit) for sg in (-1.0, 1.0) for su in (-1.0, 1.0)]
    lo, hi = np.minimum.reduce(corners), np.maximum.reduce(corners)
    ea = (2.0 * alpha * limit + 16.0) * 2.0 ** -23
    m = np.maximum(np.abs(lo), np.abs(hi))
    return h, lo - ea * m, hi + ea * m


def _scale_byte_of_amax(amax: np.ndarray) -> np.ndarray:
    """e8m0 byte the MXFP8 conversion gives a block of largest magnitude amax."""
    _, x = np.frexp(amax)
    s = np.clip(x - 9, -127, 127)
    return np.where(amax > 0, s, -127) + 127


def check_h_codes(h_ref, lo, hi, codes, scales) -> int:
    """Each GPU code and block scale of h must be one that some fp32 h in
    [lo, hi] produces: h rounded to bf16 (nearest even), then converted to
    MXFP8 (block scale from the largest magnitude, E4M3 nearest even).  A
    block whose oracle value holds a NaN must carry the NaN scale and zero
    codes.  Arrays are [n, F] (scales [n, F / 32]).  Returns how many codes
    differ from the oracle's own code of h (a count, for the report)."""
    n, F = h_ref.shape
    nb = F // 32
    nan_el = np.isnan(h_ref)
    nan_blk = nan_el.reshape(n, nb, 32).any(axis=2)
    cb = codes.reshape(n, nb, 32)
    assert np.all(scales[nan_blk] == 255) and np.all(cb[nan_blk] == 0), "NaN block of h without the NaN scale"
    fin_blk = ~nan_blk
    lo = np.where(nan_el, 0.0, lo)
    hi = np.where(nan_el, 0.0, hi)
    b_lo, b_hi = O.round_bf16(lo), O.round_bf16(hi)
    minabs = np.where((b_lo <= 0) & (b_hi >= 0), 0.0, np.minimum(np.abs(b_lo), np.abs(b_hi)))
    maxabs = np.maximum(np.abs(b_lo), np.abs(b_hi))
    s_lo = _scale_byte_of_amax(minabs.reshape(n, nb, 32).max(axis=2))
    s_hi = _scale_byte_of_amax(maxabs.reshape(n, nb, 32).max(axis=2))
    sc = scales.astype(np.int64)
    bad = fin_blk & ((sc < s_lo) | (sc > s_hi))
    assert not bad.any(), (f"{int(bad.sum())} block scales of h outside their admissible range, e.g. "
                           f"row/block {np.argwhere(bad)[:3].tolist()}: gpu {sc[bad][:3]} range {s_lo[bad][:3]}..{s_hi[bad][:3]}")
    step = np.repeat(np.ldexp(1.0, np.where(fin_blk, sc - 127, 0).astype(np.int32)), 32, axis=1)
    v_lo = O.e4m3_value(O.e4m3_encode(b_lo / step))
    v_hi = O.e4m3_value(O.e4m3_encode(b_hi / step))
    v = O.e4m3_value(codes)
    fin_el = np.repeat(fin_blk, 32, axis=1)
    bad = fin_el & ~((v >= v_lo) & (v <= v_hi))
    assert not bad.any(), (f"{int(bad.sum())} E4M3 codes of h are not admissible, e.g. at "
                           f"{np.argwhere(bad)[:3].tolist()}: gpu {v[bad][:3]} range {v_lo[bad][:3]}..{v_hi[bad][:3]}")
    own_c, own_s = O.mxfp8_quantize(np.where(nan_el, np.nan, O.round_bf16(np.where(nan_el, 0.0, h_ref))))
    return int(np.sum((own_c != codes) & fin_el))


def mx_layer_reference(w, a: dict, cfg: dict, g_idx, g_sp, wts, toks, ws: torch.Tensor):
    """For MXFP8-activation layers: check the GPU's MXFP8 codes of h for the
    rows of the sampled tokens, then return the oracle's output of those
    tokens continued from the GPU's h (and the count of codes that differ
    from the oracle's own)."""
    from mixture_experts_transformer_router_amd import moe_ffn
    assert cfg.get("act") == "clipped_swiglu", "MXFP8 activations come with the clipped SwiGLU"
    T, k, F = w.T, w.k, w.d_ff
    co, so, rb = moe_ffn.mxfp8_h_layout(T, w.d, F, w.E, k)
    P = T * k
    hq = ws[co:co + P * rb].view(P, rb)[:, :F].cpu().numpy()
    hs = ws[so:so + P * rb // 32].view(P, rb // 32)[:, :F // 32].cpu().numpy()
    pos = np.empty(P, dtype=np.int64)
    pos[g_sp] = np.arange(P)
    x = O.layer_input(a, cfg, toks)
    W = O.ExpertWeights(a, cfg["dtype"], cfg.get("weights", "dense"))
    idx = g_idx[toks]
    h_gpu = np.zeros((toks.size, k, F))
    differ = 0
    w_emin = E4M3_EMIN if cfg.get("weights") == "mxfp8" else E2M1_EMIN
    for e in np.unique(idx):
        t_sel, j_sel = np.nonzero(idx == e)
        rows = pos[toks[t_sel] * k + j_sel]
        Wg, bg, Wu, bu, _, _ = W.expert(int(e))
        xc, xs = O.mxfp8_quantize(x[t_sel])
        h, lo, hi = h_admissible_interval(
            O.mxfp8_dequantize(xc, xs), code_exponent_floor(xs, x.shape[1], E4M3_EMIN),
            Wg, code_exponent_floor(a["w_gate_scales"][e], x.shape[1], w_emin), bg,
            Wu, code_exponent_floor(a["w_up_scales"][e], x.shape[1], w_emin), bu, cfg["alpha"], cfg["limit"])
        differ += check_h_codes(h, lo, hi, hq[rows], hs[rows])
        h_gpu[t_sel, j_sel] = O.mxfp8_dequantize(hq[rows], hs[rows])
    return O.experts_forward_from_h(a, cfg, idx, wts, h_gpu), differ
