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
_GEMM_SOURCES = ["gemm_bf16.hip", "gemm_fp8.hip", "gemm_fp8_ring.hip", "gemm_simple.hip",
                 "moe_internal.h"]
KERNEL_SOURCES = {
    "gemm_gate_up": _GEMM_SOURCES,
    "gemm_down": _GEMM_SOURCES,
    "route": ["route.hip", "moe_internal.h"],
    "permute": ["permute.hip", "moe_internal.h"],
    "combine": ["combine.hip", "moe_internal.h"],
}

# device kernel names of each layer step: the grouped GEMMs take the
# epilogue (SwiGLU = gate/up) as their first template argument; the split
# tail's reduce kernel belongs to its GEMM; route and permute are one to
# three kernels per call, whose counters add up per call
KERNEL_PATTERNS = {
    "gemm_gate_up": re.compile(r"(gemm_(bf16|fp8_ring|fp8|simple)_kernel|split_reduce_kernel)<true"),
    "gemm_down": re.compile(r"(gemm_(bf16|fp8_ring|fp8|simple)_kernel|split_reduce_kernel)<false"),
    "route": re.compile(r"route_"),
    "permute": re.compile(r"perm_"),
    "combine": re.compile(r"combine_kernel"),
}
# the first kernel of each call of a step (one dispatch per call)
CALL_PATTERNS = {
    "gemm_gate_up": re.compile(r"gemm_(bf16|fp8_ring|fp8|simple)_kernel<true"),
    "gemm_down": re.compile(r"gemm_(bf16|fp8_ring|fp8|simple)_kernel<false"),
    "route": re.compile(r"route_(small|logits)"),
    "permute": re.compile(r"perm_(rank|fused)"),
    "combine": re.compile(r"combine_kernel"),
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


def per_call(csv_path: str, counter: str, kernel: str) -> list[float]:
    """Counter value of every call of a layer step: the dispatches of the
    step's kernels (KERNEL_PATTERNS), summed over their instances and over
    the kernels of one call; a call starts at its first kernel
    (CALL_PATTERNS) and takes the step's dispatches up to the next start."""
    by_disp: dict[int, list] = {}
    with open(csv_path) as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] == counter and KERNEL_PATTERNS[kernel].search(row["Kernel_Name"]):
                e = by_disp.setdefault(int(row["Dispatch_Id"]), [row["Kernel_Name"], 0.0])
                e[1] += float(row["Counter_Value"])
    calls = []
    for d in sorted(by_disp):
        name, v = by_disp[d]
        if CALL_PATTERNS[kernel].search(name) or not calls:
            calls.append(0.0)
        calls[-1] += v
    return calls


def traffic_record(fetch_csv: str, write_csv: str, kernel: str, config: str) -> dict:
    fk = per_call(fetch_csv, "FETCH_SIZE", kernel)
    wk = per_call(write_csv, "WRITE_SIZE", kernel)
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


def mfma_record(pmc_csv: str, trace_csv: str, kernel: str, config: str, xcds: int = 8,
                simds: int = 1024) -> dict:
    """Matrix-core utilisation of one GEMM step from a counter run with
    GRBM_GUI_ACTIVE, SQ_VALU_MFMA_BUSY_CYCLES and SQ_INSTS_VALU_MFMA_MOPS_*
    (plus its kernel trace for the durations): per call, the median of
      clock   = GRBM_GUI_ACTIVE (summed over the XCDs) / xcds / duration,
      util    = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / xcds * simds),
      flops   = SQ_INSTS_VALU_MFMA_MOPS_* * 512 (the MFMA work done, padding
                rows included) / duration."""
    pat = CALL_PATTERNS[kernel]
    grbm = per_dispatch(pmc_csv, "GRBM_GUI_ACTIVE", pat)
    busy = per_dispatch(pmc_csv, "SQ_VALU_MFMA_BUSY_CYCLES", pat)
    mops = []
    for c in ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_F8",
              "SQ_INSTS_VALU_MFMA_MOPS_F32"):
        v = per_dispatch(pmc_csv, c, pat)
        if v:
            mops = v
            break
    durs = []
    for r in csv.DictReader(open(trace_csv)):
        if pat.search(r["Kernel_Name"]):
            durs.append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    if not (grbm and busy and durs) or len(grbm) != len(durs):
        raise ValueError("missing or unmatched dispatches: %d counters, %d durations"
                         % (len(grbm), len(durs)))
    clk = [g / xcds / (t * 1e-9) / 1e9 for g, t in zip(grbm, durs)]
    util = [b / (g / xcds * simds) for b, g in zip(busy, grbm)]
    rec = {
        "kernel": kernel, "config": config, "source_hash": source_hash(kernel),
        "dispatches": len(durs),
        "duration_us_median": statistics.median(durs) / 1e3,
        "clock_ghz_median": round(statistics.median(clk), 4),
        "mfma_busy_fraction_median": round(statistics.median(util), 4),
        "grbm_gui_active_median": statistics.median(grbm),
        "mfma_busy_cycles_median": statistics.median(busy),
    }
    if mops and len(mops) == len(durs):
        tf = [m * 512 / (t * 1e-9) / 1e12 for m, t in zip(mops, durs)]
        rec["mfma_mops_median"] = statistics.median(mops)
        rec["mfma_tflops_median"] = round(statistics.median(tf), 2)
    return rec


def timed_averages(trace_csv: str, last: int) -> dict:
    """Average duration (ns) of the last `last` dispatches of every kernel in
    a rocprofv3 kernel_trace.csv (in dispatch order).  With bench.py run as
    `--no-configs --no-extras` and `last` = its --steps these are the timed
    loop's calls (after the per-call pass and the warm-up; the extras, when
    run, come before all of them)."""
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


TRAFFIC_COMMANDS = [
    "rocprofv3 --pmc FETCH_SIZE --kernel-include-regex \"route_|perm_|gemm_|split_reduce|combine_|"
    "stats_|copyBuffer\" --kernel-trace --output-format csv -d $OUT/FETCH_SIZE_<cfg> -o p -- "
    "python3 $REPO/bench.py --no-cpu-baseline --no-configs --no-extras --config <cfg> --steps 3 "
    "--warmup 1 --calib-copy",
    "(the same with WRITE_SIZE into $OUT/WRITE_SIZE_<cfg>)",
    "python -m grouped_gemm_router_amd.profiling --fetch $OUT/FETCH_SIZE_<cfg>/p_counter_collection.csv "
    "--write $OUT/WRITE_SIZE_<cfg>/p_counter_collection.csv --kernel <step> --config <cfg> "
    "--out profiles/traffic_<step>_<cfg>",
]


def summary(profiles_dir: str) -> str:
    """Markdown tables of every traffic_*.json and mfma_*.json record."""
    import glob
    steps = ["route", "permute", "gemm_gate_up", "gemm_down", "combine"]
    lines = ["# Counter records of the MoE layer steps", "",
             "## HBM traffic (FETCH_SIZE + WRITE_SIZE, per launch)", "",
             "Two counter runs per workload (from /tmp, `$REPO` = repository root, `$OUT` a "
             "scratch folder), then one record per step:", "", "```"] + TRAFFIC_COMMANDS + [
             "```", "",
             "Counters are KiB per dispatch, scaled by what they read for the plain 1 GiB copy "
             "that `--calib-copy` runs in the same process; the median over the 8 calls of the "
             "run (1 untimed, 3 of the per-call timing pass, 1 warm-up, 3 timed).  A step of several "
             "kernels (route, permute, a GEMM with its split-tail reduce) is summed per call.  "
             "FETCH_SIZE counts L2 misses to the memory fabric: reads served by the 256 MB MALL "
             "count too.  A record whose `source_hash` no longer matches the sources is stale.",
             "", "| Workload | Step | Fetch MB | Write MB | Total MB | source hash current |",
             "|---|---|---|---|---|---|"]
    recs = [json.load(open(f)) for f in sorted(glob.glob(os.path.join(profiles_dir, "traffic_*.json")))]
    recs.sort(key=lambda r: (r["config"], steps.index(r["kernel"])))
    for r in recs:
        lines.append("| %s | %s | %.1f | %.1f | %.1f | %s |" % (
            r["config"], r["kernel"], r["fetch_bytes_per_launch"] / 1e6,
            r["write_bytes_per_launch"] / 1e6, r["bytes_per_launch"] / 1e6,
            "yes" if r["source_hash"] == source_hash(r["kernel"]) else "no"))
    m = [json.load(open(f)) for f in sorted(glob.glob(os.path.join(profiles_dir, "mfma_*.json")))]
    if m:
        lines += ["", "## Matrix-core utilisation of the grouped GEMMs", "",
                  "One counter run per workload (command in each record), "
                  "GRBM_GUI_ACTIVE + SQ_VALU_MFMA_BUSY_CYCLES + the MFMA ops counter of the "
                  "GEMM's type; median over the run's 8 calls.  Clock = GRBM_GUI_ACTIVE / 8 XCDs "
                  "/ duration; busy = MFMA-busy cycles / (1024 SIMDs x those cycles); "
                  "TFLOP/s = MFMA ops x 512 / duration (the work the matrix cores did, "
                  "padding rows included).", "",
                  "| Workload | GEMM | Duration (us) | Clock (GHz) | MFMA busy | MFMA TFLOP/s |",
                  "|---|---|---|---|---|---|"]
        m.sort(key=lambda r: (r["config"], r["kernel"]))
        for r in m:
            lines.append("| %s | %s | %.1f | %.3f | %.3f | %s |" % (
                r["config"], r["kernel"], r["duration_us_median"], r["clock_ghz_median"],
                r["mfma_busy_fraction_median"], r.get("mfma_tflops_median", "-")))
    return "\n".join(lines) + "\n"


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
    p.add_argument("--mfma", help="counter_collection.csv of a run with the MFMA counters")
    p.add_argument("--summary", help="write the markdown summary of a profiles folder")
    p.add_argument("--config")
    p.add_argument("--out", required=True,
                   help="traffic: output path without extension (.json); trace: the .md path")
    a = p.parse_args()
    if a.summary:
        text = summary(a.summary)
        with open(a.out, "w") as f:
            f.write(text)
        print(text)
        return
    if not a.config:
        p.error("--config is required")
    if a.mfma:
        if not (a.trace and a.kernel):
            p.error("--mfma needs --trace and --kernel")
        rec = mfma_record(a.mfma, a.trace, a.kernel, a.config)
        rec["command"] = a.command or ""
        with open(a.out + ".json", "w") as f:
            json.dump(rec, f, indent=1)
        print(json.dumps(rec, indent=1))
        return
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
