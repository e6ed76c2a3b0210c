#!/usr/bin/env python3
"""Benchmark of the MoE-FFN layer on one MI355X; prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
                    [--workload decode|prefill|mxfp4|glm|tiny|block_decode|block_glm|dense_block|
                                glm_int4|glm_int8|mxfp4_mx8|mxfp8_mx8|nvfp4|mxfp4_decode]
                    [--no-prefill] [--cpu-all]

A step is one whole layer forward (route, permute, gate|up, down, combine)
over one batch of seeded synthetic tokens already resident in HBM.  The
default workload is the GPT-OSS-20B-shaped decode layer (T=8, d=d_ff=2880,
E=32, k=4, bf16): `value` is its tokens/s over the K timed steps.  The
default run also times the T=8192 prefill layer of the same shapes (the
other half of the metric: %MFMA at T=8192) and reports it under "prefill".
Expert weights rotate over several device copies so that successive steps
cannot hit the 256 MB last-level cache.  The block_* workloads run the same
layers as MoE blocks (RMSNorm in front, residual after).  mxfp4_mx8
(mxfp8_mx8) is the MXFP4 (MXFP8) layer with MXFP8 activations on the scaled
MFMA; its roofline peak is the dense fp8 MFMA rate (the E4M3 operand sets the
instruction's rate).

`roofline` reports the gate|up kernel: algorithmic bytes (few tokens) or
flops (many tokens) per launch divided by its average launch time, measured
with HIP events that the library records on the launch stream during the
timed steps.  `whole_call` divides the whole call's algorithmic bytes (or
flops) by the time of a step.  `cpu_baseline` times the float64 CPU oracle
on a bounded sample of the same workload; --cpu-all instead times it on every
workload, with all host threads and with one, and prints one JSON line per
workload (no GPU work).
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-FFN tokens/s; %HBM BW (T=8) and %MFMA peak (T=8192), E=32 k=4"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP8_PEAK_TFLOPS = 5000.0
STAGE_GATE_UP = 2
FEW_TOKEN_WORKLOADS = ("decode", "block_decode", "mxfp4_decode")
STEPS = {"decode": 500, "tiny": 500, "prefill": 50, "mxfp4": 50, "glm": 100, "block_decode": 500,
         "block_glm": 100, "dense_block": 100, "glm_int4": 100, "glm_int8": 100, "mxfp4_mx8": 50,
         "mxfp8_mx8": 50, "nvfp4": 50, "mxfp4_decode": 500}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="decode", choices=sorted(STEPS))
    ap.add_argument("--copies", type=int, default=4, help="weight copies rotated across steps")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="budget of the CPU oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true", help="skip the T=8192 prefill leg of the default run")
    ap.add_argument("--cpu-all", action="store_true",
                    help="time the CPU oracle on every workload (all threads and one thread); no GPU work")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain device copy of known size (counter calibration)")
    return ap.parse_args()


def workload(name):
    from mixture_experts_transformer_router_amd import workloads as W
    return {"decode": W.GPTOSS_DECODE, "prefill": W.GPTOSS_PREFILL, "mxfp4": W.GPTOSS_MXFP4,
            "glm": W.GLM4_MOE_LITE, "tiny": W.TINY_F32, "block_decode": W.GPTOSS_DECODE_BLOCK,
            "block_glm": W.GLM4_MOE_LITE_BLOCK, "dense_block": W.GLM4_DENSE_BLOCK,
            "glm_int4": W.GLM4_MOE_LITE_INT4, "glm_int8": W.GLM4_MOE_LITE_INT8,
            "mxfp4_mx8": W.GPTOSS_MXFP4_MX8, "mxfp8_mx8": W.GPTOSS_MXFP8_MX8, "nvfp4": W.GPTOSS_NVFP4,
            "mxfp4_decode": W.GPTOSS_MXFP4_DECODE}[name]


def matrix_bytes(w, rows, cols):
    """Bytes of one [rows, cols] expert weight matrix in w's storage format
    (codes and scales for the quantized formats)."""
    n = rows * cols
    if w.weights == "mxfp4":
        return n // 2 + n // 32
    if w.weights == "mxfp8":
        return n + n // 32
    if w.weights == "nvfp4":
        return n // 2 + n // 16
    if w.weights in ("affine4", "affine8"):
        bits, group = (4, 32) if w.weights == "affine4" else (8, 64)
        return n * bits // 8 + 2 * 2 * n // group
    return n * (2 if w.dtype == "bf16" else 4)


def expert_weight_bytes(w):
    """Bytes of one routed expert: its gate, up and down matrices and biases."""
    eb = 2 if w.dtype == "bf16" else 4
    return (2 * matrix_bytes(w, w.d_ff, w.d) + matrix_bytes(w, w.d, w.d_ff)
            + ((2 * w.d_ff + w.d) * eb if w.expert_bias else 0))


def shared_beside_router(w):
    """Whether the library runs the shared expert's tiles in the router's and
    the permutation's launches (bf16, more than 16 tokens, no RMSNorm
    prologue, at most 128 routed experts); the timed gate|up stage then holds
    the routed experts' tiles only."""
    return bool(w.d_ff_shared) and w.dtype == "bf16" and w.act_quant is None and w.T > 16 \
        and not w.block and w.E <= 128


def algorithmic_gate_up(w, counts):
    """Bytes and flops one gate|up stage must move / perform.

    bytes: gate and up weights and biases of every expert that has rows, the
    token rows (T x d) once, the hidden rows written (rows x d_ff).  flops: 2
    per multiply-add of the gate and up products.  The shared expert counts
    when its tiles run inside the timed gate|up stage (in the routed launch
    or, beside low-bit routed experts, a launch of its own), not when they
    run beside the router."""
    eb = 2 if w.dtype == "bf16" else 4
    active = [e for e, c in enumerate(counts) if c > 0]
    gu_bytes = 2 * matrix_bytes(w, w.d_ff, w.d) + (2 * w.d_ff * eb if w.expert_bias else 0)
    rows = w.P
    nbytes = len(active) * gu_bytes + w.T * w.d * eb + rows * w.d_ff * eb
    flops = 2.0 * rows * 2 * w.d_ff * w.d
    if w.d_ff_shared and not shared_beside_router(w):
        nbytes += 2 * w.d_ff_shared * w.d * eb + w.T * w.d_ff_shared * eb
        flops += 2.0 * w.T * 2 * w.d_ff_shared * w.d
    return nbytes, flops, len(active)


def algorithmic_call(w, n_active):
    """Bytes and flops of one whole layer call: every active expert's weights
    once, the router weight and bias, the token rows read and the output rows
    written; 2 flops per multiply-add of the router and the three expert
    products of every routed row (and of the shared expert)."""
    eb = 2 if w.dtype == "bf16" else 4
    nbytes = n_active * expert_weight_bytes(w) + w.E * w.d * eb + w.E * eb + 2 * w.T * w.d * eb
    flops = 2.0 * w.P * 3 * w.d * w.d_ff + 2.0 * w.T * w.d * w.E
    if w.d_ff_shared:
        nbytes += 3 * w.d_ff_shared * w.d * eb
        flops += 2.0 * w.T * 3 * w.d * w.d_ff_shared
    return nbytes, flops


def recorded_traffic(workload_name):
    """HBM bytes per launch of the gate|up kernel, from the rocprofv3
    FETCH_SIZE / WRITE_SIZE runs recorded in profiles/traffic.json
    (calibrated on a plain copy); None when none was recorded for this
    workload or the kernel's sources changed since."""
    from mixture_experts_transformer_router_amd import prof_summary as PS
    path = PS.TRAFFIC_JSON
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(workload_name)
    digest = PS.source_digest(rec["kernel"]) if rec else None
    if digest is None or rec.get("source_sha256") != digest:
        return None
    return rec["bytes"]


def host_cpu():
    """CPU model (from /proc/cpuinfo) and the number of logical CPUs this process may use."""
    model = platform.processor() or "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        nproc = len(os.sched_getaffinity(0))
    except AttributeError:
        nproc = os.cpu_count() or 1
    return model, nproc


def time_oracle(w, a, budget_s, n_tok, max_calls=50):
    """Tokens/s of the float64 oracle on the first n_tok tokens of the layer,
    repeated until budget_s has passed (or max_calls calls)."""
    import numpy as np
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from oracle import moe_oracle as O
    from parity_util import cfg_of
    cfg = cfg_of(w)
    toks = np.arange(n_tok)
    done, calls, t0 = 0, 0, time.perf_counter()
    while True:
        O.moe_layer(a, cfg, tokens=toks)
        done += n_tok
        calls += 1
        el = time.perf_counter() - t0
        if el >= budget_s or calls >= max_calls:
            return done / el, calls, el


def blas_threads():
    from threadpoolctl import threadpool_info
    return max([p.get("num_threads", 1) for p in threadpool_info()] + [1])


def cpu_baseline(w, a, budget_s):
    """Time the float64 oracle on a bounded sample of the workload."""
    model, nproc = host_cpu()
    n_tok = min(w.T, 64)
    rate, calls, el = time_oracle(w, a, budget_s, n_tok)
    return {"value": rate, "unit": "tokens/s", "cores": int(blas_threads()), "kind": "oracle",
            "cpu_model": model, "nproc": nproc,
            "sample": f"{calls} float64 oracle calls of {n_tok} tokens of the same layer "
                      f"({el:.1f} s, numpy/OpenBLAS)"}


def cpu_all(budget_s):
    """One JSON line per workload: the oracle with all BLAS threads and with one."""
    from threadpoolctl import threadpool_limits
    from mixture_experts_transformer_router_amd import inputs as I
    model, nproc = host_cpu()
    for name in ("tiny", "decode", "prefill", "mxfp4", "glm"):
        w = workload(name)
        a = I.make_inputs(w)
        n_tok = min(w.T, 64)
        rec = {"workload": w.name, "cpu_model": model, "nproc": nproc, "tokens_per_call": n_tok}
        rate, calls, el = time_oracle(w, a, budget_s, n_tok)
        rec["all_threads"] = {"threads": int(blas_threads()), "tokens_per_s": rate, "calls": calls, "s": el}
        with threadpool_limits(limits=1):
            rate, calls, el = time_oracle(w, a, budget_s, n_tok)
            rec["one_thread"] = {"threads": 1, "tokens_per_s": rate, "calls": calls, "s": el}
        print(json.dumps(rec), flush=True)


def measure(w, steps, warm, n_copies, dev="cuda"):
    """Time `steps` layer calls of workload w after `warm` untimed ones,
    rotating n_copies device copies of the weights.  Returns the timing, the
    gate|up kernel's average launch time from the library's stage events and
    the realised expert loads."""
    import numpy as np
    import torch
    from mixture_experts_transformer_router_amd import inputs as I
    from mixture_experts_transformer_router_amd import layer as LY
    from mixture_experts_transformer_router_amd import moe_ffn

    print(f"[bench] workload {w.name}: generating inputs", file=sys.stderr, flush=True)
    a = I.make_inputs(w)
    t0 = LY.to_device(a, dev)
    copies = [t0]
    weight_keys = [k for k in t0 if k not in ("x",) and isinstance(t0[k], torch.Tensor)]
    for _ in range(max(0, n_copies - 1)):
        copies.append({k: (v.clone() if k in weight_keys else v) for k, v in t0.items()})
    ws = LY.workspace_for(w, dev)
    out = torch.empty((w.T, w.d), dtype=t0["x"].dtype, device=dev)

    # routing of this batch (for the algorithmic byte count)
    _, r = LY.run(w, t0, routing=True)
    torch.cuda.synchronize()
    counts = np.diff(r["expert_offsets"].cpu().numpy())

    calls = [moe_ffn.bound_layer_call(w, c, out, ws) for c in copies]
    print(f"[bench] {w.name}: warmup {warm} steps", file=sys.stderr, flush=True)
    for i in range(warm):
        calls[i % len(calls)]()
    torch.cuda.synchronize()

    moe_ffn.profile_enable(1 << STAGE_GATE_UP)
    print(f"[bench] {w.name}: timing {steps} steps", file=sys.stderr, flush=True)
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    ev0.record(stream)
    for i in range(steps):
        calls[i % len(calls)]()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    prof = moe_ffn.profile_read()
    moe_ffn.profile_enable(0)
    gpu_ms = ev0.elapsed_time(ev1)
    gu_ms, gu_n = prof["gate_up"]
    res = {"a": a, "counts": counts, "ms_per_step": gpu_ms / steps, "tokens_per_s": w.T * steps / (gpu_ms / 1e3),
           "gate_up_s": gu_ms / max(gu_n, 1) / 1e3, "wall_s": wall, "copies": len(copies)}
    del copies, calls, out, ws
    torch.cuda.empty_cache()
    return res


def prefill_leg(args):
    """The T=8192 half of the metric: tokens/s, whole-call %MFMA and the gate|up kernel's %MFMA."""
    w = workload("prefill")
    steps = STEPS["prefill"]
    m = measure(w, steps, max(5, steps // 10), args.copies)
    nbytes_gu, flops_gu, n_active = algorithmic_gate_up(w, m["counts"])
    _, flops_call = algorithmic_call(w, n_active)
    t_call = m["ms_per_step"] / 1e3
    gu = flops_gu / m["gate_up_s"] / 1e12
    return {"workload": w.name, "T": w.T, "steps": steps, "ms_per_step": m["ms_per_step"],
            "tokens_per_s": m["tokens_per_s"],
            "whole_call": {"bound": "mfma", "achieved": flops_call / t_call / 1e12, "peak": BF16_PEAK_TFLOPS,
                           "unit": "TFLOP/s", "frac": flops_call / t_call / 1e12 / BF16_PEAK_TFLOPS},
            "gate_up_kernel": {"achieved": gu, "frac": gu / BF16_PEAK_TFLOPS, "avg_us": m["gate_up_s"] * 1e6,
                               "traffic": recorded_traffic("prefill")},
            "expert_rows_max_min": [int(m["counts"].max()), int(m["counts"].min())]}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} (WORLD_SIZE={world}) is not supported: "
              "this MoE-FFN build has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)
    if args.cpu_all:
        cpu_all(args.cpu_seconds)
        return

    import torch

    w = workload(args.workload)
    steps = args.steps or STEPS[args.workload]
    warm = args.warmup if args.warmup is not None else max(5, steps // 10)
    m = measure(w, steps, warm, args.copies)
    nbytes, flops, n_active = algorithmic_gate_up(w, m["counts"])
    call_bytes, call_flops = algorithmic_call(w, n_active)
    t_call = m["ms_per_step"] / 1e3
    gu_s = m["gate_up_s"]

    if args.workload in FEW_TOKEN_WORKLOADS:
        roof = {"bound": "hbm", "achieved": nbytes / gu_s / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
        whole = {"bound": "hbm", "achieved": call_bytes / t_call / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                 "bytes": call_bytes}
    else:
        peak = FP8_PEAK_TFLOPS if w.act_quant == "mxfp8" else BF16_PEAK_TFLOPS
        roof = {"bound": "mfma", "achieved": flops / gu_s / 1e12, "peak": peak, "unit": "TFLOP/s"}
        whole = {"bound": "mfma", "achieved": call_flops / t_call / 1e12, "peak": peak, "unit": "TFLOP/s",
                 "flops": call_flops, "hbm_GBs": call_bytes / t_call / 1e9,
                 "hbm_frac": call_bytes / t_call / 1e9 / HBM_PEAK_GBS}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = recorded_traffic(args.workload)
    roof["kernel"] = "gate_up"
    roof["kernel_avg_us"] = gu_s * 1e6
    whole["frac"] = whole["achieved"] / whole["peak"]

    prefill = None
    if args.workload == "decode" and not args.no_prefill:
        prefill = prefill_leg(args)

    if args.copy_probe:
        src = torch.empty(1 << 28, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] cpu oracle baseline", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, m["a"], args.cpu_seconds)

    line = {
        "metric": METRIC, "value": m["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": steps,
        "warmup": warm, "ms_per_step": m["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"mxfp8 x {w.weights}" if w.act_quant == "mxfp8" else w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "T": w.T, "d": w.d, "d_ff": w.d_ff, "E": w.E, "k": w.k,
                   "active_experts": n_active, "weight_copies": m["copies"], "parallelism": "none"},
        "roofline": roof, "whole_call": whole, "prefill": prefill, "cpu_baseline": cpu,
        "wall_s_timed": m["wall_s"],
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
