"""Summaries of rocprofv3 CSV output (kernel statistics and HBM counters).

    python -m mixture_experts_transformer_router_amd.prof_summary stats <kernel_stats.csv>
    python -m mixture_experts_transformer_router_amd.prof_summary pmc <fetch.csv> <write.csv> [copy_bytes]
    python -m mixture_experts_transformer_router_amd.prof_summary traffic <workload> <kernel> <fetch.csv> <write.csv>

`stats` prints a table of per-kernel call counts and durations from
`rocprofv3 --kernel-trace --stats --output-format csv`.

`traffic` records the calibrated bytes per dispatch of one kernel of one
bench workload in profiles/traffic.json, with the digest of the sources that
built it (bench.py reports the figure only while that digest still matches).

`pmc` reads two `rocprofv3 --pmc FETCH_SIZE` / `--pmc WRITE_SIZE` counter
collections (KiB per dispatch) of a run that also executed plain device
copies of `copy_bytes` bytes (bench.py --copy-probe: 256 MiB).  Each counter
is calibrated by what it reads for that copy (the copy reads and writes
exactly copy_bytes), and the per-dispatch averages of every kernel are
printed raw and calibrated, with a JSON line at the end.
"""
from __future__ import annotations

import collections
import csv
import json
import re
import sys

COPY_KERNEL = "__amd_rocclr_copyBuffer"
DEFAULT_COPY_BYTES = 1 << 28


def short_name(name: str) -> str:
    """moe::(anonymous namespace)::mfma_gemm_kernel<true, 4, 64, 2, 2>(...) -> mfma_gemm_kernel<true, 4, 64, 2, 2>"""
    n = re.sub(r"\(.*$", "", name.replace("(anonymous namespace)::", ""))
    n = n.replace("void ", "").replace("moe::", "")
    return n.strip()


def stats_table(path: str) -> str:
    rows = list(csv.DictReader(open(path)))
    out = ["| kernel | calls | avg us | min us | max us | total % |", "|---|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| {short_name(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                   f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f} |")
    return "\n".join(out)


def _per_kernel(path: str, counter: str):
    agg = collections.defaultdict(list)
    probe = []  # (dispatch id, value) of the copy kernel
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == counter:
            name = short_name(r["Kernel_Name"])
            agg[name].append(float(r["Counter_Value"]))
            if name == COPY_KERNEL:
                probe.append((int(r["Dispatch_Id"]), float(r["Counter_Value"])))
    # bench.py --copy-probe runs its 3 copies after every other GPU step
    probe.sort()
    return agg, [v for _, v in probe[-3:]]


def pmc_table(fetch_csv: str, write_csv: str, copy_bytes: int = DEFAULT_COPY_BYTES):
    f, f_probe = _per_kernel(fetch_csv, "FETCH_SIZE")
    w, w_probe = _per_kernel(write_csv, "WRITE_SIZE")
    copy_kib = copy_bytes / 1024.0
    f_copy = sum(f_probe) / len(f_probe) if f_probe else copy_kib
    w_copy = sum(w_probe) / len(w_probe) if w_probe else copy_kib
    f_scale, w_scale = copy_kib / f_copy, copy_kib / w_copy
    lines = [f"calibration: copy of {copy_bytes} B reads FETCH_SIZE {f_copy:.0f} KiB (x{f_scale:.3f}), "
             f"WRITE_SIZE {w_copy:.0f} KiB (x{w_scale:.3f})",
             "", "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | calibrated fetch MB | calibrated write MB |",
             "|---|---|---|---|---|---|"]
    result = {"fetch_scale": f_scale, "write_scale": w_scale, "kernels": {}}
    for k in sorted(set(f) | set(w)):
        if k == COPY_KERNEL:
            continue
        fv = sum(f.get(k, [0])) / max(len(f.get(k, [])), 1)
        wv = sum(w.get(k, [0])) / max(len(w.get(k, [])), 1)
        fb, wb = fv * 1024 * f_scale, wv * 1024 * w_scale
        lines.append(f"| {k} | {len(f.get(k, []))} | {fv:.0f} | {wv:.0f} | {fb / 1e6:.1f} | {wb / 1e6:.1f} |")
        result["kernels"][k] = {"fetch_kib": fv, "write_kib": wv, "bytes": fb + wb}
    return "\n".join(lines), result


import hashlib
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mixture_experts_transformer_router_amd", "csrc")
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")

# the sources each timed kernel family is built from
KERNEL_SOURCES = {
    "decode_kernel": ["expert_decode.hip"],
    "mfma_gemm_kernel": ["expert_gemm_mfma.hip", "gemm_common.h"],
    "lowbit_gemm_kernel": ["expert_gemm_lowbit.hip", "gemm_common.h"],
    "mx_gemm_kernel": ["expert_gemm_mx.hip", "gemm_common.h"],
}
COMMON_SOURCES = ["device_common.h", "moe_internal.h"]


def source_digest(kernel: str):
    """sha256 over the source files a kernel family is compiled from (None
    for a kernel this tree no longer builds)."""
    fam = next((k for k in KERNEL_SOURCES if kernel.startswith(k)), None)
    if fam is None:
        return None
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[fam] + COMMON_SOURCES:
        path = os.path.join(CSRC, f)
        if not os.path.exists(path):
            return None
        h.update(open(path, "rb").read())
    return h.hexdigest()


def record_traffic(workload: str, kernel: str, fetch_csv: str, write_csv: str):
    _, res = pmc_table(fetch_csv, write_csv)
    k = res["kernels"][kernel]
    data = json.load(open(TRAFFIC_JSON)) if os.path.exists(TRAFFIC_JSON) else {}
    data[workload] = {"kernel": kernel, "source_sha256": source_digest(kernel),
                      "fetch_bytes": k["fetch_kib"] * 1024 * res["fetch_scale"],
                      "write_bytes": k["write_kib"] * 1024 * res["write_scale"],
                      "bytes": k["bytes"], "fetch_scale": res["fetch_scale"], "write_scale": res["write_scale"]}
    with open(TRAFFIC_JSON, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
        f.write("\n")
    return data[workload]


def main(argv):
    if len(argv) >= 2 and argv[0] == "stats":
        print(stats_table(argv[1]))
    elif len(argv) >= 5 and argv[0] == "traffic":
        print(json.dumps(record_traffic(argv[1], argv[2], argv[3], argv[4])))
    elif len(argv) >= 3 and argv[0] == "pmc":
        text, res = pmc_table(argv[1], argv[2], int(argv[3]) if len(argv) > 3 else DEFAULT_COPY_BYTES)
        print(text)
        print()
        print(json.dumps(res))
    else:
        print(__doc__)
        return 2
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
