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


def test_gaps_per_stream_and_transition(tmp_path):
    rows = []
    for c in range(4):
        rows += _cycle(c * 100_000)
    rows.append(("__amd_rocclr_copyBuffer", 1, 85_000, 95_000))
    p = tmp_path / "trace.csv"
    _write_trace(p, rows)
    lines = ps.gaps(str(p), cycles=3, skip=1).splitlines()
    # stream 1: entry -> gate/up 5 us in each of the 3 cycles; gate/up ->
    # next entry 30 us twice (the last cycle's follower is outside the region)
    assert lines[0] == "stream 1: 6 kernels, idle between them 25.0 us/cycle"
    eg = [l for l in lines if "k_entry<bf16> -> k_gemv_stage<bf16, 2" in l]
    assert len(eg) == 1 and eg[0].split()[-3:] == ["3", "5.00", "5.00"]
    ge = [l for l in lines if "k_gemv_stage<bf16, 2, false> -> k_entry<bf16>" in l]
    assert len(ge) == 1 and ge[0].split()[-3:] == ["2", "30.00", "20.00"]
    # stream 2: one draft kernel per cycle, 40 us apart
    assert "stream 2: 3 kernels, idle between them 26.7 us/cycle" in lines


def _write_counters(d, rows):
    """rows: (dispatch id, kernel, grid, {counter: value})."""
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "x_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, name, grid, cs in rows:
            for c, v in cs.items():
                w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Grid_Size": grid, "Counter_Name": c,
                            "Counter_Value": v})


def test_traffic_per_kernel_and_copy_check(tmp_path):
    """Read bytes = 32 x DRAM 32-byte units (and 32/64/128 x the request
    counts), writes = 32/64 x the write requests; the copy's reading is shown
    against its known bytes; dispatches before the first cycle entry (a
    prefill) are left out; per-dispatch averages against the schedule's
    algorithmic bytes."""
    import json
    import seeded_inputs as si
    w = si.workload("4b_n8")
    copy = "__amd_rocclr_copyBuffer"
    SK1 = "void spd::k_skinny<1, 1, 16>(spd::SkinnyArgs)"
    GIB = 1 << 30
    rd = [(1, copy, 100, {"TCC_EA0_RDREQ_DRAM_32B_sum": GIB / 32, "TCC_EA0_RDREQ_32B_sum": 0,
                          "TCC_EA0_RDREQ_64B_sum": 0, "TCC_EA0_RDREQ_128B_sum": GIB / 128}),
          (2, GU, 7, {"TCC_EA0_RDREQ_DRAM_32B_sum": 9e9, "TCC_EA0_RDREQ_32B_sum": 0,
                      "TCC_EA0_RDREQ_64B_sum": 0, "TCC_EA0_RDREQ_128B_sum": 0}),       # before the cycles
          (3, "void spd::k_entry<unsigned short>(spd::Ctrl*)", 256, {"TCC_EA0_RDREQ_DRAM_32B_sum": 1}),
          (4, GU, 7, {"TCC_EA0_RDREQ_DRAM_32B_sum": 1e6, "TCC_EA0_RDREQ_32B_sum": 2e5,
                      "TCC_EA0_RDREQ_64B_sum": 1e5, "TCC_EA0_RDREQ_128B_sum": 1e5}),
          (5, GU, 7, {"TCC_EA0_RDREQ_DRAM_32B_sum": 3e6, "TCC_EA0_RDREQ_32B_sum": 0,
                      "TCC_EA0_RDREQ_64B_sum": 0, "TCC_EA0_RDREQ_128B_sum": 0}),
          # the draft o-projection and down projection: one instance, alternating
          (6, SK1, 160, {"TCC_EA0_RDREQ_DRAM_32B_sum": 1e5}),
          (7, SK1, 160, {"TCC_EA0_RDREQ_DRAM_32B_sum": 4e5}),
          (8, SK1, 160, {"TCC_EA0_RDREQ_DRAM_32B_sum": 3e5}),
          (9, SK1, 160, {"TCC_EA0_RDREQ_DRAM_32B_sum": 6e5})]
    red = "void at::native::reduce_kernel<512, 1, at::native::ReduceOp<float, at::native::func_wrapper_t<float, at::native::sum_functor<float, float, float>::operator()(at::TensorIterator&)::{lambda(float, float)#1}>, unsigned int, float, 4, 4> >(at::native::ReduceOp<float, at::native::func_wrapper_t<float, at::native::sum_functor<float, float, float>::operator()(at::TensorIterator&)::{lambda(float, float)#1}>, unsigned int, float, 4, 4>)"
    fill = "void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<float>, std::array<char*, 1ul> >(int, at::native::FillFunctor<float>, std::array<char*, 1ul>)"
    rd.insert(0, (0, red, 100, {"TCC_EA0_RDREQ_DRAM_32B_sum": GIB / 32 * 1.01, "TCC_EA0_RDREQ_32B_sum": 0,
                               "TCC_EA0_RDREQ_64B_sum": GIB / 64, "TCC_EA0_RDREQ_128B_sum": 0}))
    mul = "void at::native::vectorized_elementwise_kernel<4, at::native::AUnaryFunctor<float, float, float, at::native::binary_internal::MulFunctor<float> >, std::array<char*, 2ul> >(int, at::native::AUnaryFunctor<float, float, float, at::native::binary_internal::MulFunctor<float> >, std::array<char*, 2ul>)"
    rd.insert(1, (-1, mul, 100, {"TCC_EA0_RDREQ_DRAM_32B_sum": GIB / 32, "TCC_EA0_RDREQ_32B_sum": 0,
                               "TCC_EA0_RDREQ_64B_sum": 0, "TCC_EA0_RDREQ_128B_sum": GIB / 128}))
    wr = [(0, fill, 100, {"TCC_EA0_WRREQ_sum": GIB / 64, "TCC_EA0_WRREQ_64B_sum": GIB / 128}),
          (-1, mul, 100, {"TCC_EA0_WRREQ_sum": GIB / 64, "TCC_EA0_WRREQ_64B_sum": GIB / 64}),
          (1, copy, 100, {"TCC_EA0_WRREQ_sum": GIB / 64, "TCC_EA0_WRREQ_64B_sum": GIB / 64}),
          (4, GU, 7, {"TCC_EA0_WRREQ_sum": 10, "TCC_EA0_WRREQ_64B_sum": 4}),
          (5, GU, 7, {"TCC_EA0_WRREQ_sum": 10, "TCC_EA0_WRREQ_64B_sum": 4})]
    # weight generation before the calibration: a larger fill and scaling
    # (1.45 GiB) must not be taken for the calibration dispatches
    rd.insert(0, (-9, mul, 100, {"TCC_EA0_RDREQ_DRAM_32B_sum": 1.45 * GIB / 32}))
    wr.insert(0, (-9, mul, 100, {"TCC_EA0_WRREQ_sum": 1.45 * GIB / 64, "TCC_EA0_WRREQ_64B_sum": 1.45 * GIB / 64}))
    wr.insert(0, (-8, fill, 100, {"TCC_EA0_WRREQ_sum": 1.45 * GIB / 64, "TCC_EA0_WRREQ_64B_sum": 1.45 * GIB / 64}))
    _write_counters(tmp_path / "r", rd)
    _write_counters(tmp_path / "w", wr)
    sched = {"workload": "4b_n8", "cycles": [{"occupancy": 4, "exit_pos": -1}, {"occupancy": 8, "exit_pos": 5}]}
    json.dump(sched, open(tmp_path / "s.json", "w"))
    rec = ps.traffic(str(tmp_path / "r"), str(tmp_path / "w"), str(tmp_path / "s.json"))
    assert rec["sum_read"][0] == pytest.approx(1.01 * GIB) and rec["sum_read"][1] == pytest.approx(GIB)
    assert rec["fill_write"] == pytest.approx(GIB * 0.75)  # half the requests 32-byte, half 64-byte
    assert rec["ecopy_read"][0] == pytest.approx(GIB) and rec["ecopy_write"] == pytest.approx(GIB)
    table = ps.traffic_table(rec)
    assert "elementwise copy (1 GiB read + 1 GiB written): DRAM reads 1.000x" in table
    assert "sum over 1 GiB: DRAM reads 1.010x" in table and "writes 0.750x" in table
    gu = next(k for k in rec["kernels"] if k["kernel"] == "stage gate/up")
    assert gu["dispatches"] == 2
    assert gu["read_dram_bytes"] == pytest.approx(2e6 * 32)
    assert gu["read_all_bytes"] == pytest.approx((2e5 * 32 + 1e5 * 64 + 1e5 * 128) / 2)
    assert gu["write_bytes"] == pytest.approx(6 * 32 + 4 * 64)
    assert gu["algorithmic_bytes"] == pytest.approx(6 * 2 * w.F * w.d * 2)  # mean occupancy 6
    assert rec["traffic_bytes_per_launch"] == pytest.approx(2e6 * 32 + 6 * 32 + 4 * 64)
    assert rec["source_hash"] == ps.kernel_source_hash()
    o = next(k for k in rec["kernels"] if k["kernel"] == "draft o-projection")
    dn = next(k for k in rec["kernels"] if k["kernel"] == "draft down")
    assert o["dispatches"] == dn["dispatches"] == 2
    assert o["read_dram_bytes"] == pytest.approx(2e5 * 32) and dn["read_dram_bytes"] == pytest.approx(5e5 * 32)
    assert o["algorithmic_bytes"] == pytest.approx(w.Hq * w.hd * w.d * 2)
    assert dn["algorithmic_bytes"] == pytest.approx(w.d * w.F * 2)
    assert "stage gate/up" in ps.traffic_table(rec)


def test_bench_reports_only_a_current_traffic_record():
    """bench.py reports the counted traffic only while the record's source
    hash matches the GEMV sources (a kernel change since the counters were
    taken makes it report none)."""
    import json
    import bench
    rec = json.load(open(ps.TRAFFIC_JSON))
    got = bench.traffic_bytes(rec.get("workload"))
    if rec.get("source_hash") == ps.kernel_source_hash():
        assert got == int(rec["traffic_bytes_per_launch"]) and got > 0
    else:
        assert got is None
    assert bench.traffic_bytes("another workload") is None


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
