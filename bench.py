#!/usr/bin/env python3
"""Benchmark of the MoE-FFN layer on one MI355X; prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
                    [--workload decode|prefill|mxfp4|glm|tiny|block_decode|block_glm|dense_block|
                                glm_int4|glm_int8|mxfp4_mx8|mxfp8_mx8|nvfp4|mxfp4_decode]

A step is one whole layer forward (route, permute, gate|up, down, combine)
over one batch of seeded synthetic tokens already resident in HBM.  The
default workload is the GPT-OSS-20B-shaped decode layer (T=8, d=d_ff=2880,
E=32, k=4, bf16).  Expert weights rotate over several device copies so that
successive steps cannot hit the 256 MB last-level cache.  The block_*
workloads run the same layers as MoE blocks (RMSNorm in front, residual
after).  mxfp4_mx8 (mxfp8_mx8) is the MXFP4 (MXFP8) layer with MXFP8 activations on the
scaled MFMA; its roofline peak is the dense fp8 MFMA rate (the E4M3 operand
sets the instruction's rate).

`value` is tokens/s over the K timed steps.  `roofline` reports the gate|up
kernel: algorithmic bytes (decode) or flops (prefill) per launch divided by
its average launch time, measured with HIP events that the library records
on the launch stream during the timed steps.  `cpu_baseline` times the
float64 CPU oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-FFN tokens/s; %HBM BW (T=8) and %MFMA peak (T=8192), E=32 k=4"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP8_PEAK_TFLOPS = 5000.0
STAGE_GATE_UP = 2


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="decode",
                    choices=["decode", "prefill", "mxfp4", "glm", "tiny", "block_decode", "block_glm",
                             "dense_block", "glm_int4", "glm_int8", "mxfp4_mx8", "mxfp8_mx8", "nvfp4",
                             "mxfp4_decode"])
    ap.add_argument("--copies", type=int, default=4, help="weight copies rotated across steps")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="budget of the CPU oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
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


def shared_beside(w):
    """True when a shared expert's GEMMs run on the library's second stream,
    beside the routed gate|up launch that the stage timer measures (bf16
    shared expert, more tokens than the weight-streaming path takes)."""
    return bool(w.d_ff_shared) and w.T > 16 and w.dtype == "bf16"


def algorithmic_gate_up(w, counts):
    """Bytes and flops one gate|up launch must move / perform.

    bytes: weights and biases of every expert that has rows, the token rows
    (T x d) once, the hidden rows written (rows x d_ff).  flops: 2 per
    multiply-add of the gate and up products.  The shared expert counts only
    when its tiles are in the timed launch."""
    eb = 2 if w.dtype == "bf16" else 4
    active = [e for e, c in enumerate(counts) if c > 0]
    if w.weights == "mxfp4":
        wbytes_per_expert = 2 * (w.d_ff * w.d // 2 + w.d_ff * w.d // 32)
    elif w.weights == "mxfp8":
        wbytes_per_expert = 2 * (w.d_ff * w.d + w.d_ff * w.d // 32)
    elif w.weights == "nvfp4":
        wbytes_per_expert = 2 * (w.d_ff * w.d // 2 + w.d_ff * w.d // 16)
    elif w.weights in ("affine4", "affine8"):
        bits, group = (4, 32) if w.weights == "affine4" else (8, 64)
        wbytes_per_expert = 2 * (w.d_ff * w.d * bits // 8 + 2 * 2 * w.d_ff * w.d // group)
    else:
        wbytes_per_expert = 2 * w.d_ff * w.d * eb
    bias = 2 * w.d_ff * eb if w.expert_bias else 0
    rows = w.P
    nbytes = len(active) * (wbytes_per_expert + bias) + w.T * w.d * eb + rows * w.d_ff * eb
    flops = 2.0 * rows * 2 * w.d_ff * w.d
    if w.d_ff_shared and not shared_beside(w):
        nbytes += 2 * w.d_ff_shared * w.d * eb + w.T * w.d_ff_shared * eb
        flops += 2.0 * w.T * 2 * w.d_ff_shared * w.d
    return nbytes, flops, len(active)


def recorded_traffic(w, workload_name):
    """HBM bytes per launch of the gate|up kernel, from the rocprofv3
    FETCH_SIZE / WRITE_SIZE runs recorded in profiles/traffic.json
    (calibrated on a plain copy); None when none was recorded for this
    workload or the kernel's sources changed since."""
    import json
    from mixture_experts_transformer_router_amd import prof_summary as PS
    path = PS.TRAFFIC_JSON
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(workload_name)
    digest = PS.source_digest(rec["kernel"]) if rec else None
    if digest is None or rec.get("source_sha256") != digest:
        return None
    return rec["bytes"]


def cpu_baseline(w, a, budget_s):
    """Time the float64 oracle on a bounded sample of the workload."""
    import numpy as np
    from threadpoolctl import threadpool_info
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from oracle import moe_oracle as O
    from parity_util import cfg_of
    cfg = cfg_of(w)
    n_tok = min(w.T, 64)
    toks = np.arange(n_tok)
    done, t0 = 0, time.perf_counter()
    calls = 0
    while True:
        O.moe_layer(a, cfg, tokens=toks)
        done += n_tok
        calls += 1
        el = time.perf_counter() - t0
        if el >= budget_s or calls >= 50:
            break
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {"value": done / el, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{calls} float64 oracle calls of {n_tok} tokens of the same layer "
                      f"({el:.1f} s, numpy/OpenBLAS)"}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} (WORLD_SIZE={world}) is not supported: "
              "this MoE-FFN build has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from mixture_experts_transformer_router_amd import inputs as I
    from mixture_experts_transformer_router_amd import layer as LY
    from mixture_experts_transformer_router_amd import moe_ffn

    w = workload(args.workload)
    steps = args.steps or {"decode": 500, "tiny": 500, "prefill": 50, "mxfp4": 50, "glm": 100,
                           "block_decode": 500, "block_glm": 100, "dense_block": 100, "glm_int4": 100,
                           "glm_int8": 100, "mxfp4_mx8": 50, "mxfp8_mx8": 50, "nvfp4": 50,
                           "mxfp4_decode": 500}[args.workload]
    warm = args.warmup if args.warmup is not None else max(5, steps // 10)
    dev = "cuda"
    print(f"[bench] workload {w.name}: generating inputs", file=sys.stderr, flush=True)
    a = I.make_inputs(w)
    t0 = LY.to_device(a, dev)
    copies = [t0]
    weight_keys = [k for k in t0 if k not in ("x",) and isinstance(t0[k], torch.Tensor)]
    for _ in range(max(0, args.copies - 1)):
        copies.append({k: (v.clone() if k in weight_keys else v) for k, v in t0.items()})
    ws = LY.workspace_for(w, dev)
    out = torch.empty((w.T, w.d), dtype=t0["x"].dtype, device=dev)

    # routing of this batch (for the algorithmic byte count)
    _, r = LY.run(w, t0, routing=True)
    torch.cuda.synchronize()
    offs = r["expert_offsets"].cpu().numpy()
    counts = np.diff(offs)
    nbytes, flops, n_active = algorithmic_gate_up(w, counts)

    calls = [moe_ffn.bound_layer_call(w, c, out, ws) for c in copies]
    print(f"[bench] warmup {warm} steps", file=sys.stderr, flush=True)
    for i in range(warm):
        calls[i % len(calls)]()
    torch.cuda.synchronize()

    moe_ffn.profile_enable(1 << STAGE_GATE_UP)
    print(f"[bench] timing {steps} steps", file=sys.stderr, flush=True)
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
    ms_per_step = gpu_ms / steps
    value = w.T * steps / (gpu_ms / 1e3)

    gu_ms, gu_n = prof["gate_up"]
    gu_avg_s = gu_ms / max(gu_n, 1) / 1e3
    if args.workload in ("decode", "block_decode", "mxfp4_decode"):
        roof = {"bound": "hbm", "achieved": nbytes / gu_avg_s / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    else:
        peak = FP8_PEAK_TFLOPS if w.act_quant == "mxfp8" else BF16_PEAK_TFLOPS
        roof = {"bound": "mfma", "achieved": flops / gu_avg_s / 1e12, "peak": peak, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = recorded_traffic(w, args.workload)
    roof["kernel"] = "gate_up (routed experts; the shared expert runs beside it)" if shared_beside(w) else "gate_up"
    roof["kernel_avg_us"] = gu_avg_s * 1e6

    if args.copy_probe:
        src = torch.empty(1 << 28, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] cpu oracle baseline", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, a, args.cpu_seconds)

    line = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": steps, "warmup": warm,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": f"mxfp8 x {w.weights}" if w.act_quant == "mxfp8" else w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "T": w.T, "d": w.d, "d_ff": w.d_ff, "E": w.E, "k": w.k,
                   "active_experts": n_active, "weight_copies": len(copies), "parallelism": "none"},
        "roofline": roof, "cpu_baseline": cpu,
        "wall_s_timed": wall,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
