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


def _multi_csv(path, rows):
    """rows: (dispatch id, kernel name, counter, value, start ns, end ns)"""
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=COUNTER_FIELDS, quoting=csv.QUOTE_NONNUMERIC)
        w.writeheader()
        for d, name, c, v, t0, t1 in rows:
            r = {k: 0 for k in COUNTER_FIELDS}
            r.update(Correlation_Id=d, Dispatch_Id=d, Kernel_Name=name, Counter_Name=c,
                     Counter_Value=v, Agent_Id="Agent 1", Start_Timestamp=t0, End_Timestamp=t1)
            w.writerow(r)


def test_counters_derive_busy_clock_instructions_and_bytes(tmp_path):
    # a 2 x 2 x 2 grid of "chip": 2 CUs x 4 SIMDs, 2 XCDs; one dispatch of 1000 ns
    # with 3200 cycles summed over the 2 XCDs (1600 per XCD -> 1.6 GHz), MFMA
    # busy 6400 of 8 x 1600 SIMD-cycles (0.5), 100 MFMA instructions against a
    # closed form of 2^17 FLOP / 1024 per instruction = 128
    p1 = tmp_path / "p1.csv"
    _multi_csv(p1, [(1, GEMM, "GRBM_GUI_ACTIVE", 3200, 0, 1000),
                    (1, GEMM, "SQ_VALU_MFMA_BUSY_CYCLES", 6400, 0, 1000),
                    (1, GEMM, "SQ_INSTS_VALU_MFMA_F16", 100, 0, 1000),
                    (1, GEMM, "SQ_BUSY_CU_CYCLES", 2400, 0, 1000)])
    # second pass: FETCH / WRITE with a 1 MiB copy reading 512 KiB (factor 2)
    p2 = tmp_path / "p2.csv"
    _multi_csv(p2, [(1, COPY, "FETCH_SIZE", 512, 0, 50), (1, COPY, "WRITE_SIZE", 1024, 0, 50),
                    (2, GEMM, "FETCH_SIZE", 10, 0, 2000), (2, GEMM, "WRITE_SIZE", 5, 0, 2000),
                    (2, GEMM, "SQ_LDS_BANK_CONFLICT", 30, 0, 2000),
                    (2, GEMM, "SQ_LDS_IDX_ACTIVE", 120, 0, 2000),
                    (2, GEMM, "TCC_HIT_sum", 3, 0, 2000), (2, GEMM, "TCC_MISS_sum", 1, 0, 2000),
                    (2, GEMM, "TCC_EA0_RDREQ_sum", 8, 0, 2000),
                    (2, GEMM, "TCC_EA0_RDREQ_DRAM_sum", 2, 0, 2000)])
    out = tmp_path / "c.md"
    assert rs.main(["counters", "--pmc", str(p1), "--command", "c1", "--pmc", str(p2),
                    "--command", "c2", "--title", "t", "--out", str(out), "--cus", "2",
                    "--xcds", "2", "--flop", str(1 << 17), "--mfma-flop", "1024",
                    "--copy-bytes", str(1 << 20), "--algo-bytes", str(30 * 1024)]) == 0
    text = open(out).read()
    assert "    c1\n    c2" in text
    assert "| GPU cycles per dispatch | 1600 |" in text
    assert "| effective clock | 1.600 GHz |" in text  # from the GRBM pass (1000 ns)
    assert "| MFMA busy | 0.500 |" in text
    # 2400 busy cycles over 2 CUs: 1200 per CU, 1.2 GHz, MFMA busy 6400 / (8 x 1200)
    assert "| busy cycles per CU | 1200 |" in text
    assert "| clock while busy | 1.200 GHz |" in text
    assert "| MFMA busy per busy CU cycle | 0.667 |" in text
    assert "| MFMA instructions / closed form | 100 / 128 = 0.7812 |" in text
    assert "| LDS bank-conflict share | 0.2500 |" in text
    assert "| L2 hit rate | 0.750 |" in text
    assert "| L2 read requests to DRAM | 0.250 |" in text
    assert "| HBM read bytes | 2.048e+04 |" in text and "| HBM write bytes | 5120 |" in text
    assert "| traffic / algorithmic bytes | 0.833 |" in text
    # the copy is not a library kernel and gets no table of its own
    assert "## `%s`" % COPY not in text


def test_counters_need_one_command_per_pass(tmp_path):
    p1 = tmp_path / "p1.csv"
    _multi_csv(p1, [(1, GEMM, "GRBM_GUI_ACTIVE", 1, 0, 1)])
    with pytest.raises(SystemExit):
        rs.main(["counters", "--pmc", str(p1), "--pmc", str(p1), "--command", "c",
                 "--title", "t", "--out", str(tmp_path / "x.md")])


def test_traffic_adds_the_kernels_of_one_launch(tmp_path):
    # a split-K launch: the GEMM kernel and the reduce kernel, one dispatch each
    red = "void libgemm::splitk_reduce_kernel<float>(Params)"
    fetch = [(1, COPY, 1024.0), (2, GEMM, 100.0), (3, red, 30.0)]
    write = [(1, COPY, 1024.0), (2, GEMM, 40.0), (3, red, 10.0)]
    t = _traffic(tmp_path, fetch, write)
    assert t["fetch_size_kib"] == 130.0 and t["write_size_kib"] == 50.0
    assert t["kernels"] == sorted([GEMM, red])


def test_stats_rate_per_launch(tmp_path):
    # a split-K launch: the GEMM kernel (2000 ns) and its reduce (500 ns)
    path = tmp_path / "s.csv"
    with open(path, "w", newline="") as f:
        w = csv.writer(f, quoting=csv.QUOTE_NONNUMERIC)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs",
                    "MaxNs", "StdDev"])
        w.writerow([GEMM, 10, 20000, 2000.0, 70.0, 1900, 2100, 1.0])
        w.writerow(["void libgemm::splitk_reduce_kernel(Params)", 10, 5000, 500.0, 20.0, 400,
                    600, 1.0])
        w.writerow(["other", 1, 100, 100.0, 10.0, 100, 100, 0.0])
    out = tmp_path / "s.md"
    assert rs.main(["stats", "--csv", str(path), "--command", "x", "--out", str(out),
                    "--bytes", "10000000", "--flop", "5000000000"]) == 0
    text = open(out).read()
    assert "| 10 | 2.00 | 1.90 | 2.10 | 70.0 |" in text
    # 2500 ns per launch: 1e7 B -> 4000 GB/s, 5e9 FLOP -> 2000 TFLOP/s
    assert "2.50 us, 2000.0 TFLOP/s (5000000000 FLOP), 4000.0 GB/s" in text
