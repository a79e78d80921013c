"""CPU tests of the rocprofv3 summary tool that produces the committed traffic
and kernel-time figures, on small synthetic CSV files in rocprofv3's format."""
from __future__ import annotations

import csv
import json

import pytest

from dense_mixed_precision_tiled_amd import rocprof_summary as rs

COUNTER_FIELDS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id",
                  "Thread_Id", "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size",
                  "LDS_Block_Size", "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count",
                  "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp",
                  "End_Timestamp"]
GEMM = "void libgemm::gemm_mfma_kernel<libgemm::TileCfg<256, 256, 64, 2, 4, 32, 2, 1>>(Params)"
COPY = "__amd_rocclr_copyBuffer"


def _counter_csv(path, counter, rows):
    """rows: (dispatch id, kernel name, value); several rows of one dispatch are
    counter instances that the tool must add up."""
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=COUNTER_FIELDS, quoting=csv.QUOTE_NONNUMERIC)
        w.writeheader()
        for d, name, v in rows:
            r = {k: 0 for k in COUNTER_FIELDS}
            r.update(Correlation_Id=d, Dispatch_Id=d, Kernel_Name=name, Counter_Name=counter,
                     Counter_Value=v, Agent_Id="Agent 1")
            w.writerow(r)


def _traffic(tmp_path, fetch_rows, write_rows, copy_bytes=1 << 20):
    _counter_csv(tmp_path / "f.csv", "FETCH_SIZE", fetch_rows)
    _counter_csv(tmp_path / "w.csv", "WRITE_SIZE", write_rows)
    out = tmp_path / "t.json"
    rc = rs.main(["traffic", "--fetch", str(tmp_path / "f.csv"), "--write",
                  str(tmp_path / "w.csv"), "--copy-bytes", str(copy_bytes), "--command", "cmd",
                  "--out", str(out)])
    assert rc == 0
    return json.load(open(out))


def test_traffic_calibrates_by_the_copy_and_takes_the_median_dispatch(tmp_path):
    # a 1 MiB copy reads 512 KiB by the counter (factor 2) and writes 1024 KiB
    # (factor 1); the GEMM dispatches read 100, 300, 200 KiB (median 200) and
    # write 50 KiB; an unrelated kernel is ignored
    fetch = [(1, "other_kernel", 9999.0), (2, COPY, 512.0), (3, GEMM, 100.0),
             (4, GEMM, 300.0), (5, GEMM, 200.0)]
    write = [(1, COPY, 1024.0), (2, GEMM, 50.0), (3, GEMM, 50.0)]
    t = _traffic(tmp_path, fetch, write)
    assert t["fetch_factor"] == pytest.approx(2.0)
    assert t["write_factor"] == pytest.approx(1.0)
    assert t["fetch_size_kib"] == 200.0 and t["write_size_kib"] == 50.0
    assert t["read_bytes"] == pytest.approx(200 * 1024 * 2.0)
    assert t["write_bytes"] == pytest.approx(50 * 1024 * 1.0)
    assert t["bytes_per_launch"] == pytest.approx(t["read_bytes"] + t["write_bytes"])
    assert t["copy_kernel"] == COPY and t["command"] == "cmd"
    assert t["kernel_source_hash"] == rs.kernel_source_hash()


def test_counter_instances_of_one_dispatch_are_summed(tmp_path):
    # dispatch 3 reports its FETCH_SIZE in two instances (60 + 40 KiB)
    fetch = [(2, COPY, 1024.0), (3, GEMM, 60.0), (3, GEMM, 40.0)]
    write = [(1, COPY, 1024.0), (2, GEMM, 10.0)]
    t = _traffic(tmp_path, fetch, write)
    assert t["fetch_size_kib"] == 100.0


def test_traffic_needs_both_the_gemm_and_the_copy(tmp_path):
    with pytest.raises(SystemExit):
        _traffic(tmp_path, [(3, GEMM, 1.0)], [(1, COPY, 1.0), (2, GEMM, 1.0)])


def test_stats_table_in_microseconds(tmp_path):
    path = tmp_path / "s.csv"
    long_name = "k" * 200
    with open(path, "w", newline="") as f:
        w = csv.writer(f, quoting=csv.QUOTE_NONNUMERIC)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs",
                    "MaxNs", "StdDev"])
        w.writerow([GEMM, 110, 15227883, 138435.3, 99.5, 126105, 235452, 1.0])
        w.writerow([long_name, 1, 3920, 3920.0, 0.5, 3920, 3920, 0.0])
    out = tmp_path / "s.md"
    assert rs.main(["stats", "--csv", str(path), "--command", "rocprofv3 ...",
                    "--out", str(out)]) == 0
    text = open(out).read()
    assert "    rocprofv3 ..." in text
    assert "| 110 | 138.44 | 126.11 | 235.45 | 99.5 |" in text
    # long kernel names are cut to 110 characters, ending in "..."
    assert "`" + "k" * 107 + "...`" in text


def test_source_hash_is_stable_and_short():
    h = rs.kernel_source_hash()
    assert h == rs.kernel_source_hash() and len(h) == 16
    int(h, 16)
