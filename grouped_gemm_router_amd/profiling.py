"""Summaries of rocprofv3 runs for profiles/: the HBM traffic of one kernel
from counter passes, and a per-kernel table of a kernel trace.

HBM traffic.

Two `rocprofv3 --pmc` runs of `bench.py --calib-copy` (one with FETCH_SIZE,
one with WRITE_SIZE; the counters are KiB per dispatch) give the bytes a
kernel pulls from and pushes to HBM.  Each counter is scaled by what it reads
for the plain 1 GiB device copy that `--calib-copy` runs in the same process
(1 GiB read, 1 GiB written), so the record is in the same units as the
algorithmic bytes.  The record carries a hash of the kernel sources; bench.py
uses it only while the sources are unchanged.

    python -m grouped_gemm_router_amd.profiling \\
        --fetch <dir>/f_counter_collection.csv --write <dir>/w_counter_collection.csv \\
        --kernel gemm_gate_up --config mixtral_bf16 --out profiles/traffic_gemm_gate_up_mixtral_bf16

Kernel trace.  `--stats <dir>/<cfg>_kernel_stats.csv` (from `rocprofv3
--kernel-trace --stats`) becomes a markdown table of the layer's kernels
(calls, average / min / max duration); the kernels that generate the
synthetic inputs are summed into one line.

    python -m grouped_gemm_router_amd.profiling --stats <dir>/mixtral_bf16_kernel_stats.csv \\
        --config mixtral_bf16 --command "<the rocprofv3 command>" \\
        --out profiles/kernel_trace_moe_layer_mixtral_bf16.md
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
import statistics

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "grouped_gemm_router_amd", "csrc")

# kernel sources whose change invalidates a traffic record
KERNEL_SOURCES = {
    "gemm_gate_up": ["gemm_bf16.hip", "gemm_fp8.hip", "gemm_fp8_ring.hip", "gemm_simple.hip",
                     "moe_internal.h"],
    "gemm_down": ["gemm_bf16.hip", "gemm_fp8.hip", "gemm_fp8_ring.hip", "gemm_simple.hip",
                  "moe_internal.h"],
}

# device kernel names: the grouped GEMMs take the epilogue (SwiGLU = gate/up)
# as their first template argument
KERNEL_PATTERNS = {
    "gemm_gate_up": re.compile(r"gemm_(bf16|fp8_ring|fp8|simple)_kernel<true"),
    "gemm_down": re.compile(r"gemm_(bf16|fp8_ring|fp8|simple)_kernel<false"),
}
COPY_PATTERN = re.compile(r"copyBuffer")
COPY_BYTES = 1 << 30


def source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for n in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def per_dispatch(csv_path: str, counter: str, pattern) -> list[float]:
    """Counter value (summed over its instances) of every matching dispatch."""
    vals: dict[str, float] = {}
    with open(csv_path) as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] != counter or not pattern.search(row["Kernel_Name"]):
                continue
            key = row["Dispatch_Id"]
            vals[key] = vals.get(key, 0.0) + float(row["Counter_Value"])
    return [vals[k] for k in sorted(vals, key=int)]


def traffic_record(fetch_csv: str, write_csv: str, kernel: str, config: str) -> dict:
    pat = KERNEL_PATTERNS[kernel]
    fk = per_dispatch(fetch_csv, "FETCH_SIZE", pat)
    wk = per_dispatch(write_csv, "WRITE_SIZE", pat)
    fc = per_dispatch(fetch_csv, "FETCH_SIZE", COPY_PATTERN)
    wc = per_dispatch(write_csv, "WRITE_SIZE", COPY_PATTERN)
    if not (fk and wk and fc and wc):
        raise ValueError("missing dispatches: kernel %d/%d, copy %d/%d"
                         % (len(fk), len(wk), len(fc), len(wc)))
    # the largest copy dispatch is the 1 GiB calibration copy
    f_scale = COPY_BYTES / max(fc)
    w_scale = COPY_BYTES / max(wc)
    fetch = statistics.median(fk) * f_scale
    write = statistics.median(wk) * w_scale
    return {
        "kernel": kernel,
        "config": config,
        "source_hash": source_hash(kernel),
        "fetch_bytes_per_launch": round(fetch),
        "write_bytes_per_launch": round(write),
        "bytes_per_launch": round(fetch + write),
        "dispatches": [len(fk), len(wk)],
        "fetch_kib_median": statistics.median(fk),
        "write_kib_median": statistics.median(wk),
        "copy_fetch_kib": max(fc),
        "copy_write_kib": max(wc),
        "bytes_per_counter_unit": [f_scale, w_scale],
    }


# kernels of this library (everything else in a bench trace generates inputs)
LIBRARY_KERNELS = re.compile(r"route_|perm_|gemm_|split_reduce|combine_|stats_|quantize")


def timed_averages(trace_csv: str, last: int) -> dict:
    """Average duration (ns) of the last `last` dispatches of every kernel in
    a rocprofv3 kernel_trace.csv (in dispatch order): the timed steps of a
    bench run, without its warm-up calls."""
    per = {}
    for r in csv.DictReader(open(trace_csv)):
        per.setdefault(r["Kernel_Name"], []).append(
            (int(r["Dispatch_Id"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    out = {}
    for name, v in per.items():
        v.sort()
        tail = [d for _, d in v[-last:]]
        out[name] = sum(tail) / len(tail)
    return out


def trace_summary(stats_csv: str, config: str, command: str, trace_csv: str = None,
                  timed: int = 0) -> str:
    """Markdown table of a rocprofv3 kernel_stats.csv; with the matching
    kernel_trace.csv, also the average over the last `timed` calls."""
    rows = list(csv.DictReader(open(stats_csv)))
    tavg = timed_averages(trace_csv, timed) if trace_csv and timed > 0 else None
    lines = ["# Kernel trace: MoE layer step, %s" % config, "",
             "Command (from /tmp, `$REPO` = repository root, one MI355X):", "",
             "```", command, "```", ""]
    if tavg is not None:
        lines += ["'Timed avg' is the mean of each kernel's last %d calls (the bench's timed "
                  "steps, without the warm-up calls run before the clocks settle); it is the "
                  "figure to compare with the bench's per-kernel HIP-event times." % timed, "",
                  "| Kernel | Calls | Avg (us) | Timed avg (us) | Min (us) | Max (us) |",
                  "|---|---|---|---|---|---|"]
    else:
        lines += ["| Kernel | Calls | Avg (us) | Min (us) | Max (us) |", "|---|---|---|---|---|"]
    other_calls, other_ns = 0, 0.0
    for r in rows:
        name = r["Name"].replace("(anonymous namespace)::", "").replace("void ", "")
        if not LIBRARY_KERNELS.search(name.split("(")[0]):
            other_calls += int(r["Calls"])
            other_ns += float(r["TotalDurationNs"])
            continue
        if tavg is not None:
            lines.append("| `%s` | %s | %.2f | %.2f | %.2f | %.2f |" % (
                name.split("(")[0], r["Calls"], float(r["AverageNs"]) / 1e3,
                tavg.get(r["Name"], float("nan")) / 1e3, float(r["MinNs"]) / 1e3,
                float(r["MaxNs"]) / 1e3))
        else:
            lines.append("| `%s` | %s | %.2f | %.2f | %.2f |" % (
                name.split("(")[0], r["Calls"], float(r["AverageNs"]) / 1e3,
                float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3))
    lines += ["", "Input generation and copies outside the layer (torch kernels): %d calls, "
              "%.1f ms in total." % (other_calls, other_ns / 1e6), ""]
    return "\n".join(lines)


def main() -> None:
    p = argparse.ArgumentParser()
    p.add_argument("--fetch", help="counter_collection.csv of the FETCH_SIZE pass")
    p.add_argument("--write", help="counter_collection.csv of the WRITE_SIZE pass")
    p.add_argument("--kernel", choices=sorted(KERNEL_PATTERNS))
    p.add_argument("--stats", help="kernel_stats.csv of a kernel trace")
    p.add_argument("--command", help="the rocprofv3 command of the trace")
    p.add_argument("--trace", help="kernel_trace.csv of the same run (per dispatch)")
    p.add_argument("--timed", type=int, default=0,
                   help="with --trace: average the last this many calls of each kernel")
    p.add_argument("--config", required=True)
    p.add_argument("--out", required=True,
                   help="traffic: output path without extension (.json); trace: the .md path")
    a = p.parse_args()
    if a.stats:
        text = trace_summary(a.stats, a.config, a.command or "", a.trace, a.timed)
        with open(a.out, "w") as f:
            f.write(text)
        print(text)
        return
    if not (a.fetch and a.write and a.kernel):
        p.error("traffic needs --fetch, --write and --kernel")
    rec = traffic_record(a.fetch, a.write, a.kernel, a.config)
    with open(a.out + ".json", "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec, indent=1))


if __name__ == "__main__":
    main()
