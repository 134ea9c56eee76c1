"""The rocprofv3 summary tool on small synthetic traces and counter files:
per-stream busy time, device-idle time and per-kernel averages of a
timeline, and the copy-calibrated HBM traffic of the gate/up GEMV."""
import csv
import os

import pytest

from pipelined_draft_verify_amd import profile_summary as ps

TRACE_FIELDS = ["Kernel_Name", "Stream_Id", "Start_Timestamp", "End_Timestamp", "Grid_Size_X", "Grid_Size_Y",
                "Grid_Size_Z"]
GU = "void spd::k_gemv_stage<unsigned short, 2, false>(spd::StageGemv)"


def _write_trace(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=TRACE_FIELDS)
        w.writeheader()
        for name, st, t0, t1 in rows:
            w.writerow({"Kernel_Name": name, "Stream_Id": st, "Start_Timestamp": t0, "End_Timestamp": t1,
                        "Grid_Size_X": 256, "Grid_Size_Y": 1, "Grid_Size_Z": 1})


def _cycle(c0):
    """One 100 us cycle (ns timestamps): entry and gate/up on stream 1, a
    draft kernel on stream 2 overlapping gate/up, 20 us with no kernel."""
    return [("void spd::k_entry<unsigned short>(spd::Ctrl*)", 1, c0, c0 + 5_000),
            (GU, 1, c0 + 10_000, c0 + 70_000),
            ("void spd::k_mfma_gemv<2, 1, 256>(spd::MfmaArgs)", 2, c0 + 20_000, c0 + 80_000)]


def test_timeline_busy_idle_and_averages(tmp_path):
    rows = []
    for c in range(4):
        rows += _cycle(c * 100_000)
    # a host-side copy between steps is not part of the region
    rows.append(("__amd_rocclr_copyBuffer", 1, 85_000, 95_000))
    p = tmp_path / "trace.csv"
    _write_trace(p, rows)
    out = ps.timeline(str(p), cycles=3, skip=1)
    lines = out.splitlines()
    # cycles 0..2: from the first entry to the last kernel end before cycle 3
    assert lines[0] == "region: 9 dispatches over 0.3 ms for 3 cycles -> 93.3 us/cycle"
    assert "stream 1: busy 0.2 ms (65.0 us/cycle)" in lines
    assert "stream 2: busy 0.2 ms (60.0 us/cycle)" in lines
    # idle: 5..10 us of every cycle and 80..100 us between cycles (the region
    # ends with the last cycle's kernels at 280 us): 55 us over 3 cycles
    assert "device idle: 18.3 us/cycle (19.6% of the region)" in lines
    gu = [l for l in lines if "k_gemv_stage<bf16, 2" in l]
    assert len(gu) == 1 and gu[0].split()[-3:] == ["3", "60.00", "60.00"]


def test_timeline_needs_enough_cycles(tmp_path):
    p = tmp_path / "trace.csv"
    _write_trace(p, _cycle(0))
    with pytest.raises(ValueError):
        ps.timeline(str(p), cycles=2)


def _write_counters(d, counter, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "x_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, v in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": v})


def test_traffic_is_scaled_by_the_calibration_copy(tmp_path):
    copy = "__amd_rocclr_copyBuffer"
    # the copy reads 1 GiB but the counter shows half: fetch scale 2
    _write_counters(tmp_path / "f", "FETCH_SIZE", [(GU, 100.0), (GU, 300.0), (copy, 4.0), (copy, 524288.0)])
    _write_counters(tmp_path / "w", "WRITE_SIZE", [(GU, 10.0), (GU, 10.0), (copy, 1048576.0)])
    rec = ps.traffic(str(tmp_path / "f"), str(tmp_path / "w"))
    assert rec["dispatches"] == [2, 2]
    assert rec["fetch_scale"] == pytest.approx(2.0) and rec["write_scale"] == pytest.approx(1.0)
    assert rec["traffic_bytes_per_launch"] == pytest.approx(200 * 1024 * 2.0 + 10 * 1024)
    assert rec["source_hash"] == ps.kernel_source_hash()


def test_committed_traffic_record_matches_the_kernel_sources():
    """bench.py reports the counted traffic only while the record's source
    hash matches the GEMV sources; the committed record must be current."""
    import json
    rec = json.load(open(ps.TRAFFIC_JSON))
    assert rec["source_hash"] == ps.kernel_source_hash()
    assert rec["traffic_bytes_per_launch"] > 0


def test_mfma_summary_counts_only_the_cycles(tmp_path):
    """Dispatches before the first k_entry (prefill) are left out; per kernel
    and grid the mean utilisation, operations per call and rate."""
    d = tmp_path / "m"
    os.makedirs(d)
    fields = ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value", "Start_Timestamp",
              "End_Timestamp"]
    mm = "void spd::k_mfma_gemv<2, 1, 256>(spd::MfmaArgs)"
    rows = [(1, mm, 77824, 50.0, 9e9, 0, 10_000),                       # prefill: ignored
            (2, "void spd::k_entry<unsigned short>(spd::Ctrl*)", 256, 0.0, 0.0, 20_000, 25_000),
            (3, mm, 77824, 2.0, 3e9, 30_000, 60_000),
            (4, mm, 77824, 4.0, 3e9, 70_000, 100_000)]
    with open(d / "m_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for i, name, grid, util, flops, t0, t1 in rows:
            for cn, cv in [("MfmaUtil", util), ("MfmaFlopsBF16", flops)]:
                w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Grid_Size": grid, "Counter_Name": cn,
                            "Counter_Value": cv, "Start_Timestamp": t0, "End_Timestamp": t1})
    lines = ps.mfma(str(d)).splitlines()
    assert len(lines) == 2
    # 2 calls, util (2 + 4) / 2 = 3 %, 3 GFLOP each over 30 us = 100 TFLOP/s = 0.04 of 2.5 PFLOP/s
    assert lines[1].split() == ["k_mfma_gemv<2,", "1,", "256>", "77824", "2", "3.00", "3.000", "30.00", "100.0",
                                "0.0400"]
