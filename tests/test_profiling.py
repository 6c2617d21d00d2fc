"""CPU checks of the profile summaries built from rocprofv3 CSVs.  Traffic
record: the kernel and copy dispatches are told apart by name, counters are
summed over their instances per dispatch, and the copy calibration scales
KiB to bytes.  Trace summary: the timed column averages each kernel's last
dispatches in dispatch order."""
import csv
import json

import pytest

from grouped_gemm_router_amd import profiling

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def write_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for d, name, vals in rows:
            for v in vals:   # one row per counter instance (e.g. per XCD)
                w.writerow({"Dispatch_Id": d, "Kernel_Name": name, "Counter_Name": counter,
                            "Counter_Value": v})


def test_traffic_record(tmp_path):
    gate = "void (anonymous namespace)::gemm_bf16_kernel<true, false, 8>(...)"
    down = "void (anonymous namespace)::gemm_bf16_kernel<false, true, 4>(...)"
    copy = "__amd_rocclr_copyBuffer"
    # the copy reads 1 GiB = 2^20 KiB but the counter shows 2^20 * 1.25
    # (so one unit is 0.8 KiB); the gate/up kernel shows 1000 units per launch
    f = tmp_path / "f.csv"
    w = tmp_path / "w.csv"
    write_csv(f, "FETCH_SIZE", [(1, gate, [600, 400]), (2, down, [5, 5]), (3, gate, [500, 500]),
                                (4, copy, [2 ** 20 * 1.25 / 2] * 2), (5, copy, [10])])
    write_csv(w, "WRITE_SIZE", [(1, gate, [100]), (2, down, [1]), (3, gate, [100]),
                                (4, copy, [2 ** 20])])
    rec = profiling.traffic_record(str(f), str(w), "gemm_gate_up", "mixtral_bf16")
    assert rec["dispatches"] == [2, 2]
    assert rec["fetch_bytes_per_launch"] == round(1000 * 0.8 * 1024)
    assert rec["write_bytes_per_launch"] == 100 * 1024
    assert rec["bytes_per_launch"] == rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"]
    assert rec["source_hash"] == profiling.source_hash("gemm_gate_up")
    json.dumps(rec)


def test_timed_averages_take_the_last_calls_in_dispatch_order(tmp_path):
    """The 'timed' column averages each kernel's last N dispatches (ordered by
    dispatch id, not file order), so warm-up calls are left out."""
    trace = tmp_path / "x_kernel_trace.csv"
    rows = [("gemm_a", 5, 0, 900), ("gemm_a", 1, 0, 5000), ("gemm_a", 3, 0, 1000),
            ("gemm_a", 7, 0, 1100), ("combine_b", 2, 10, 40), ("combine_b", 6, 10, 30)]
    with open(trace, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Dispatch_Id", "Start_Timestamp", "End_Timestamp"])
        for name, disp, t0, t1 in rows:
            w.writerow([name, disp, t0, t1])
    avg = profiling.timed_averages(str(trace), 3)
    assert avg["gemm_a"] == pytest.approx((1000 + 900 + 1100) / 3)  # dispatches 3, 5, 7
    assert avg["combine_b"] == pytest.approx((30 + 20) / 2)        # fewer calls than asked


def test_trace_summary_timed_column(tmp_path):
    stats = tmp_path / "x_kernel_stats.csv"
    trace = tmp_path / "x_kernel_trace.csv"
    with open(stats, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs",
                    "StdDev"])
        w.writerow(["void gemm_bf16_kernel<true>(int)", 3, 6000, 2000, 100, 1000, 4000, 0])
    with open(trace, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Dispatch_Id", "Start_Timestamp", "End_Timestamp"])
        for disp, dur in [(1, 4000), (2, 1000), (3, 1000)]:
            w.writerow(["void gemm_bf16_kernel<true>(int)", disp, 0, dur])
    text = profiling.trace_summary(str(stats), "cfg", "cmd", str(trace), 2)
    assert "| Timed avg (us) |" in text
    assert "| `gemm_bf16_kernel<true>` | 3 | 2.00 | 1.00 | 1.00 | 4.00 |" in text
