"""Host-only checks of the rocprofv3 summary helpers on hand-written CSV."""

import csv
import os

from grouped_quadratic_softmax_amd import profiling as P


def _write(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "x_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (k, c, v) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": k, "Counter_Name": c, "Counter_Value": v})


def test_traffic_sums_the_kernels_of_one_call(tmp_path):
    # a call that launches two kernels; the copy reads and writes 1024 KiB
    # but its counters read 512 (fetch) and 1024 (write) KiB
    _write(tmp_path / "f", [("oal::k_sums(x)", "FETCH_SIZE", 10), ("oal::k_sums(x)", "FETCH_SIZE", 12),
                            ("oal::k_out(x)", "FETCH_SIZE", 100), ("other", "FETCH_SIZE", 1e6)])
    _write(tmp_path / "w", [("oal::k_sums(x)", "WRITE_SIZE", 4), ("oal::k_out(x)", "WRITE_SIZE", 50)])
    _write(tmp_path / "cf", [("copy_kernel", "FETCH_SIZE", 512)])
    _write(tmp_path / "cw", [("copy_kernel", "WRITE_SIZE", 1024)])
    rec = P.traffic_record(str(tmp_path / "f"), str(tmp_path / "w"), str(tmp_path / "cf"), str(tmp_path / "cw"),
                           "oal::k_", 1024 * 1024, [], sources=["oal_ceilings.hip"])
    assert rec["fetch_factor"] == 2.0 and rec["write_factor"] == 1.0
    assert rec["fetch_bytes"] == (11 + 100) * 1024 * 2.0  # median of the first kernel's two dispatches
    assert rec["write_bytes"] == (4 + 50) * 1024
    assert rec["bytes_per_launch"] == rec["fetch_bytes"] + rec["write_bytes"]
    assert rec["source_sha256"] == P.source_hash(["oal_ceilings.hip"]) != P.source_hash()


def test_counters_table(tmp_path):
    _write(tmp_path / "a", [("oal::k_out(x)", "SQ_BUSY_CYCLES", 7), ("oal::k_out(x)", "SQ_BUSY_CYCLES", 9)])
    md = P.counters_markdown([str(tmp_path / "a")], ["k_out"], "t", ["cmd"])
    assert "| `oal::k_out` | 2 | 8 |" in md
