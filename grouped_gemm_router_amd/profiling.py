"""HBM traffic of one kernel from rocprofv3 counter passes.

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


def main() -> None:
    p = argparse.ArgumentParser()
    p.add_argument("--fetch", required=True, help="counter_collection.csv of the FETCH_SIZE pass")
    p.add_argument("--write", required=True, help="counter_collection.csv of the WRITE_SIZE pass")
    p.add_argument("--kernel", required=True, choices=sorted(KERNEL_PATTERNS))
    p.add_argument("--config", required=True)
    p.add_argument("--out", required=True, help="output path without extension (.json + .md)")
    a = p.parse_args()
    rec = traffic_record(a.fetch, a.write, a.kernel, a.config)
    with open(a.out + ".json", "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec, indent=1))


if __name__ == "__main__":
    main()
