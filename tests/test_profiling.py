"""CPU checks of the profile summaries built from rocprofv3 CSVs.  Traffic
record: the kernel and copy dispatches are told apart by name, counters are
summed over their instances per dispatch and over the kernels of one call of
a step, and the copy calibration scales KiB to bytes.  MFMA record: clock,
busy fraction and MFMA rate from the counters and durations.  Trace summary:
the timed column averages each kernel's last dispatches in dispatch
order."""
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


def test_traffic_of_a_multi_kernel_step(tmp_path):
    """A permutation call is three kernels (rank, scan, scatter) and a GEMM
    call may add its split tail's reduce kernel: the counters of one call add
    up, other steps' kernels in between are left out."""
    rank, scan = "perm_rank_kernel<2>(...)", "perm_scan_kernel(...)"
    scat, route = "perm_scatter_kernel<2, false>(...)", "route_small_bf16<1, 8>(...)"
    gate, red = "gemm_bf16_kernel<true, false, 8>(...)", "split_reduce_kernel<true, false>(...)"
    copy = "__amd_rocclr_copyBuffer"
    rows = []
    d = 0
    for call in range(3):
        for name, v in [(route, 7), (rank, 1), (scan, 2), (scat, 100 + call), (gate, 1000),
                        (red, 10)]:
            d += 1
            rows.append((d, name, [v / 2, v / 2]))
    rows.append((d + 1, copy, [2 ** 20]))
    f = tmp_path / "f.csv"
    w = tmp_path / "w.csv"
    write_csv(f, "FETCH_SIZE", rows)
    write_csv(w, "WRITE_SIZE", rows)
    assert profiling.per_call(str(f), "FETCH_SIZE", "permute") == [103, 104, 105]
    assert profiling.per_call(str(f), "FETCH_SIZE", "gemm_gate_up") == [1010] * 3
    assert profiling.per_call(str(f), "FETCH_SIZE", "route") == [7] * 3
    rec = profiling.traffic_record(str(f), str(w), "permute", "mixtral_bf16")
    assert rec["fetch_bytes_per_launch"] == 104 * 1024 and rec["dispatches"] == [3, 3]


def test_mfma_record(tmp_path):
    """clock = GRBM_GUI_ACTIVE / XCDs / duration; busy fraction = MFMA busy
    cycles / (cycles x SIMDs); rate = MOPS x 512 / duration."""
    gate = "gemm_bf16_kernel<true, false, 8>(...)"
    pmc = tmp_path / "p.csv"
    with open(pmc, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=FIELDS)
        wr.writeheader()
        for disp in (1, 2):
            for counter, vals in [("GRBM_GUI_ACTIVE", [2.0e6] * 8),
                                  ("SQ_VALU_MFMA_BUSY_CYCLES", [0.7 * 2.0e6 * 1024]),
                                  ("SQ_INSTS_VALU_MFMA_MOPS_BF16", [1.0e9])]:
                for v in vals:
                    wr.writerow({"Dispatch_Id": disp, "Kernel_Name": gate,
                                 "Counter_Name": counter, "Counter_Value": v})
    trace = tmp_path / "t.csv"
    with open(trace, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Dispatch_Id", "Start_Timestamp", "End_Timestamp"])
        for disp in (1, 2):
            w.writerow([gate, disp, 0, 1_000_000])   # 1 ms
    rec = profiling.mfma_record(str(pmc), str(trace), "gemm_gate_up", "mixtral_bf16")
    assert rec["clock_ghz_median"] == pytest.approx(2.0)
    assert rec["mfma_busy_fraction_median"] == pytest.approx(0.7)
    assert rec["mfma_tflops_median"] == pytest.approx(512.0)


def test_summary_tables(tmp_path):
    """The summary lists every traffic and MFMA record, in MB, steps in layer
    order, and marks a record whose source hash no longer matches."""
    rec = {"kernel": "combine", "config": "mixtral_bf16", "source_hash": "stale",
           "fetch_bytes_per_launch": 134_800_000, "write_bytes_per_launch": 33_600_000,
           "bytes_per_launch": 168_400_000}
    (tmp_path / "traffic_combine_mixtral_bf16.json").write_text(json.dumps(rec))
    rec2 = dict(rec, kernel="route", source_hash=profiling.source_hash("route"),
                fetch_bytes_per_launch=34_100_000, write_bytes_per_launch=100_000,
                bytes_per_launch=34_200_000)
    (tmp_path / "traffic_route_mixtral_bf16.json").write_text(json.dumps(rec2))
    m = {"kernel": "gemm_gate_up", "config": "mixtral_bf16", "duration_us_median": 1587.9,
         "clock_ghz_median": 1.703, "mfma_busy_fraction_median": 0.691,
         "mfma_tflops_median": 1225.94}
    (tmp_path / "mfma_gemm_gate_up_mixtral_bf16.json").write_text(json.dumps(m))
    text = profiling.summary(str(tmp_path))
    rows = [l for l in text.splitlines() if l.startswith("| mixtral_bf16")]
    assert rows[0] == "| mixtral_bf16 | route | 34.1 | 0.1 | 34.2 | yes |"
    assert rows[1] == "| mixtral_bf16 | combine | 134.8 | 33.6 | 168.4 | no |"
    assert rows[2] == "| mixtral_bf16 | gemm_gate_up | 1587.9 | 1.703 | 0.691 | 1225.94 |"


def test_one_launch_permute_calls_are_counted_apart(tmp_path):
    """The one-launch permutation kernel starts a call of its own, so its
    dispatches are not summed into one."""
    fused = "perm_fused_kernel<2, false>(...)"
    rows = [(d + 1, fused, [50.0 + d, 50.0]) for d in range(4)]
    f = tmp_path / "f.csv"
    write_csv(f, "FETCH_SIZE", rows)
    assert profiling.per_call(str(f), "FETCH_SIZE", "permute") == [100, 101, 102, 103]
