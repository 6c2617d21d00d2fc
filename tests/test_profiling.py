"""CPU checks of the traffic record built from rocprofv3 counter CSVs: the
kernel and copy dispatches are told apart by name, counters are summed over
their instances per dispatch, and the copy calibration scales KiB to bytes."""
import csv
import json

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
