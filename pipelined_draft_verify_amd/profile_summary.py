"""Summaries of rocprofv3 output for the committed profiles/ files.

  python -m pipelined_draft_verify_amd.profile_summary stats <kernel_stats.csv> [--cmd "..."]
  python -m pipelined_draft_verify_amd.profile_summary timeline <kernel_trace.csv> --cycles K [--skip S] [--cmd "..."]
  python -m pipelined_draft_verify_amd.profile_summary gaps <kernel_trace.csv> --cycles K [--skip S] [--cmd "..."]
  python -m pipelined_draft_verify_amd.profile_summary traffic <fetch_dir> <write_dir> --cmd "..."
  python -m pipelined_draft_verify_amd.profile_summary mfma <counter_dir> [--cmd "..."]

`timeline` takes K cycles of a kernel trace, ending --skip cycles before its
end (a cycle starts at each k_entry or k_tree_entry dispatch), and prints, per stream and per kernel/grid, the launches,
average duration and time per cycle, plus each stream's busy time and the
device-idle time (no kernel on any stream).

`gaps` takes the same cycles and prints, per stream, the idle time between
consecutive kernels of that stream (start of one minus end of the one before),
summed per transition (kernel -> next kernel): launch gaps inside a graph,
waits on the other stream, and waits on the host when it enqueues slower
than the GPU runs.

`traffic` reads two counter-collection runs of one workload step -- reads:
TCC_EA0_RDREQ_DRAM_32B_sum (32-byte units of L2-to-memory read requests bound
for DRAM; a 64-byte request counts 2, a 128-byte one 4) with the 32/64/128-byte
request counts TCC_EA0_RDREQ_{32B,64B,128B}_sum; writes: TCC_EA0_WRREQ_sum and
TCC_EA0_WRREQ_64B_sum (32- or 64-byte requests) -- checks them on plain
dispatches of known size (a sum over 1 GiB reads it once, a fill of 1 GiB
writes it once, an elementwise 1 GiB copy does both), and prints, per cycle
kernel, the
counted bytes per dispatch against the algorithmic bytes per dispatch of the
step's schedule (bench.py --dump-schedule).  The gate/up record (with a hash
of the kernel sources) feeds bench.py's roofline `traffic`, reported only
while that hash still matches.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic_gate_up_4b_n8.json")
GU_REGEX = r"k_gemv_stage<unsigned short, 2[,>]"
ENTRY_REGEX = r"k_(tree_)?entry<"  # the first kernel of every cycle (single chain or draft tree)
SUM_REGEX = r"reduce_kernel"
ECOPY_REGEX = r"MulFunctor"  # the elementwise copy x * 1
FILL_REGEX = r"FillFunctor"
COPY_BYTES = 1 << 30


def kernel_source_hash() -> str:
    """Hash of the code (comments and blank space removed) of the sources the
    gate/up GEMV is built from: a comment edit keeps a counter record valid,
    any code change invalidates it."""
    h = hashlib.sha256()
    for name in ("common.h", "gemv.h"):
        src = open(os.path.join(HERE, "csrc", name)).read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()[:16]


def _short(name: str) -> str:
    n = name.replace("void spd::", "").replace("spd::", "").replace("unsigned short", "bf16")
    m = re.match(r"([\w:]+)(<[^>]*>)?", n)
    return (m.group(1) + (m.group(2) or "")) if m else n[:60]


def stats(path: str, top: int = 16) -> str:
    rows = list(csv.DictReader(open(path)))
    tot = sum(float(r["TotalDurationNs"]) for r in rows)
    out = [f"{'kernel':44s} {'calls':>7s} {'avg us':>9s} {'total ms':>9s} {'%':>6s}"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"]))[:top]:
        out.append(f"{_short(r['Name'])[:44]:44s} {int(r['Calls']):7d} {float(r['AverageNs']) / 1e3:9.2f} "
                   f"{float(r['TotalDurationNs']) / 1e6:9.1f} {100 * float(r['TotalDurationNs']) / tot:6.1f}")
    return "\n".join(out)


def _region(path: str, cycles: int, skip: int):
    """Dispatches of cycles [-(cycles + skip), -skip) of the trace, in start
    order; host-side copies between steps (rollback) are not part of it."""
    rows = sorted(csv.DictReader(open(path)), key=lambda r: int(r["Start_Timestamp"]))
    ent = [i for i, r in enumerate(rows) if re.search(ENTRY_REGEX, r["Kernel_Name"])]
    if len(ent) < cycles + skip:
        raise ValueError(f"trace has {len(ent)} cycles, fewer than {cycles + skip}")
    lo = ent[-(cycles + skip)]
    hi = ent[-skip] if skip else len(rows)
    return [r for r in rows[lo:hi] if "copyBuffer" not in r["Kernel_Name"]]


def timeline(path: str, cycles: int, skip: int = 0, top: int = 30) -> str:
    sel = _region(path, cycles, skip)
    t0 = int(sel[0]["Start_Timestamp"])
    t1 = max(int(r["End_Timestamp"]) for r in sel)
    span = (t1 - t0) / 1e3
    out = [f"region: {len(sel)} dispatches over {span / 1e3:.1f} ms for {cycles} cycles "
           f"-> {span / cycles:.1f} us/cycle"]
    busy, agg = {}, {}
    for r in sel:
        d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        st = r["Stream_Id"]
        busy[st] = busy.get(st, 0.0) + d
        key = (st, _short(r["Kernel_Name"]), r["Grid_Size_X"], r["Grid_Size_Y"], r["Grid_Size_Z"])
        a = agg.setdefault(key, [0, 0.0])
        a[0] += 1
        a[1] += d
    for st in sorted(busy):
        out.append(f"stream {st}: busy {busy[st] / 1e3:.1f} ms ({busy[st] / cycles:.1f} us/cycle)")
    # device-idle: time covered by no kernel of any stream
    iv = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in sel)
    idle, end = 0, iv[0][0]
    for s0, e0 in iv:
        if s0 > end:
            idle += s0 - end
        end = max(end, e0)
    out.append(f"device idle: {idle / 1e3 / cycles:.1f} us/cycle ({100 * idle / 1e3 / span:.1f}% of the region)")
    out.append(f"{'stream':>6s} {'kernel':34s} {'grid (threads x, y, z)':>24s} {'calls':>6s} {'avg us':>8s} {'us/cycle':>9s}")
    for (st, name, gx, gy, gz), (n, t) in sorted(agg.items(), key=lambda kv: -kv[1][1])[:top]:
        out.append(f"{st:>6s} {name[:34]:34s} {gx + ',' + gy + ',' + gz:>24s} {n:6d} {t / n:8.2f} {t / cycles:9.2f}")
    return "\n".join(out)


def gaps(path: str, cycles: int, skip: int = 0, top: int = 12) -> str:
    sel = _region(path, cycles, skip)
    out = []
    per_stream = {}
    for r in sel:
        per_stream.setdefault(r["Stream_Id"], []).append(r)
    for st in sorted(per_stream):
        ks = per_stream[st]
        agg = {}
        for a, b in zip(ks, ks[1:]):
            g = (int(b["Start_Timestamp"]) - int(a["End_Timestamp"])) / 1e3
            e = agg.setdefault((_short(a["Kernel_Name"]), _short(b["Kernel_Name"])), [0, 0.0])
            e[0] += 1
            e[1] += max(g, 0.0)
        tot = sum(v[1] for v in agg.values())
        out.append(f"stream {st}: {len(ks)} kernels, idle between them {tot / cycles:.1f} us/cycle")
        out.append(f"  {'kernel -> next kernel':72s} {'count':>6s} {'mean us':>8s} {'us/cycle':>9s}")
        for (a, b), (n, t) in sorted(agg.items(), key=lambda kv: -kv[1][1])[:top]:
            out.append(f"  {(a[:34] + ' -> ' + b[:34]):72s} {n:6d} {t / n:8.2f} {t / cycles:9.2f}")
    return "\n".join(out)


def _counter_rows(d: str):
    files = glob.glob(os.path.join(d, "**", "*counter_collection*.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection csv under {d}")
    for f in files:
        yield from csv.DictReader(open(f))


def counter_values(d: str, counter: str, regex: str):
    return [float(r["Counter_Value"]) for r in _counter_rows(d)
            if r.get("Counter_Name") == counter and re.search(regex, r.get("Kernel_Name", ""))]


def counter_avg(d: str, counter: str, regex: str):
    vals = counter_values(d, counter, regex)
    return (sum(vals) / len(vals), len(vals)) if vals else (None, 0)


RD_COUNTERS = ("TCC_EA0_RDREQ_DRAM_32B_sum", "TCC_EA0_RDREQ_32B_sum", "TCC_EA0_RDREQ_64B_sum",
               "TCC_EA0_RDREQ_128B_sum")
WR_COUNTERS = ("TCC_EA0_WRREQ_sum", "TCC_EA0_WRREQ_64B_sum")


def _per_dispatch(d: str):
    """{dispatch id: {"name", "grid", counter: value}} of one counter run."""
    per = {}
    for r in _counter_rows(d):
        e = per.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"], "grid": int(r["Grid_Size"])})
        e[r["Counter_Name"]] = e.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return per


def _read_bytes(e):
    return (e.get("TCC_EA0_RDREQ_DRAM_32B_sum", 0.0) * 32.0,
            e.get("TCC_EA0_RDREQ_32B_sum", 0.0) * 32.0 + e.get("TCC_EA0_RDREQ_64B_sum", 0.0) * 64.0
            + e.get("TCC_EA0_RDREQ_128B_sum", 0.0) * 128.0)


def _write_bytes(e):
    n, n64 = e.get("TCC_EA0_WRREQ_sum", 0.0), e.get("TCC_EA0_WRREQ_64B_sum", 0.0)
    return (n - n64) * 32.0 + n64 * 64.0


def cycle_kernels(w, sched):
    """(label, kernel regex, which, algorithmic bytes per dispatch) of the
    cycle kernels of one step with the given schedule (per-cycle occupancy
    and exit).  Stage kernels stream a * matrix per launch (one launch per
    sub-step); the heads share one kernel instance (the draft head every
    cycle, the verification head launched every cycle but streaming only when
    a token exits); the draft module's products stream their matrix once per
    launch -- its o-projection and down projection share one kernel instance
    and grid and alternate within each layer (which = 0 / 1: the even / odd
    dispatches of that instance)."""
    es = 2 if w.dtype == "bf16" else 4
    d, F, V = w.d, w.F, w.V
    qkv = (w.Hq + 2 * w.Hkv) * w.hd * d * es
    wo = w.Hq * w.hd * d * es
    wgu, wdn = 2 * F * d * es, d * F * es
    K = len(sched)
    occ = sum(c["occupancy"] for c in sched) / K
    exits = sum(1 for c in sched if c["exit_pos"] >= 0)
    head = V * d * es * (K + exits) / (2 * K)
    ks = [
        ("stage q/k/v", r"k_gemv_stage<[^,]+, 0, false", None, occ * qkv),
        ("stage o-projection", r"k_gemv_stage<[^,]+, 1, false", None, occ * wo),
        ("stage gate/up", r"k_gemv_stage<[^,]+, 2, false", None, occ * wgu),
        ("stage down", r"k_gemv_stage<[^,]+, 1, true", None, occ * wdn),
        ("LM heads (draft every cycle, target on exit)", r"k_gemv_stage<[^,]+, 3, false", None, head),
        ("draft gate/up", r"k_skinny<2, ", None, wgu),
        ("draft o-projection", r"k_skinny<1, ", 0, wo),
        ("draft down", r"k_skinny<1, ", 1, wdn),
        ("draft q/k/v", r"k_skinny<0, ", None, qkv),
    ]
    return ks


def traffic(read_dir: str, write_dir: str, sched_json: str):
    """Counted read/write bytes per dispatch of each cycle kernel (dispatches
    after the first cycle entry), the copy's reading, and the ratios."""
    import seeded_inputs as si

    sc = json.load(open(sched_json))
    w = si.workload(sc["workload"])
    sched = sc["cycles"]
    rd, wr = _per_dispatch(read_dir), _per_dispatch(write_dir)
    out = {"workload": w.name, "source_hash": kernel_source_hash(), "kernels": []}
    # calibration dispatches: bench.py issues them after generating the
    # weights (whose own fills, scalings and copies match the same kernel
    # names) and before the engine's first kernel -- the last dispatch of each
    # kind before the first spd:: kernel
    for key, per, fn, rx in (("sum_read", rd, _read_bytes, SUM_REGEX), ("fill_write", wr, _write_bytes, FILL_REGEX),
                             ("ecopy_read", rd, _read_bytes, ECOPY_REGEX),
                             ("ecopy_write", wr, _write_bytes, ECOPY_REGEX)):
        ids = sorted(per)
        eng0 = next((i for i in ids if "spd::" in per[i]["name"]), None)
        cps = [i for i in ids if (eng0 is None or i < eng0) and re.search(rx, per[i]["name"])]
        if cps:
            out[key] = fn(per[cps[-1]])
    ids_r = sorted(rd)
    first = next((i for i in ids_r if re.search(ENTRY_REGEX, rd[i]["name"])), 0)
    for label, rx, which, alg in cycle_kernels(w, sched):
        sel = [i for i in ids_r if i >= first and re.search(rx, rd[i]["name"])]
        if which is not None:
            sel = sel[which::2]
        if not sel:
            continue
        r_dram = sum(_read_bytes(rd[i])[0] for i in sel) / len(sel)
        r_all = sum(_read_bytes(rd[i])[1] for i in sel) / len(sel)
        wsel = [i for i in sorted(wr) if re.search(rx, wr[i]["name"]) and i in rd and i >= first]
        wb = sum(_write_bytes(wr[i]) for i in wsel) / len(wsel) if wsel else None
        out["kernels"].append({"kernel": label, "dispatches": len(sel), "algorithmic_bytes": alg,
                               "read_dram_bytes": r_dram, "read_all_bytes": r_all, "write_bytes": wb,
                               "read_ratio": r_dram / alg if alg else None})
    gu = next((k for k in out["kernels"] if k["kernel"] == "stage gate/up"), None)
    if gu:
        out["kernel"] = "k_gemv_stage<bf16,SWIGLU>"
        out["traffic_bytes_per_launch"] = gu["read_dram_bytes"] + (gu["write_bytes"] or 0.0)
    return out


def traffic_table(rec) -> str:
    lines = []
    sr, fw = rec.get("sum_read"), rec.get("fill_write")
    if sr or fw:
        lines.append(f"calibration sum over 1 GiB: DRAM reads {sr[0] / COPY_BYTES:.3f}x, all reads "
                     f"{sr[1] / COPY_BYTES:.3f}x; fill of 1 GiB: writes {(fw or 0) / COPY_BYTES:.3f}x of the known bytes"
                     if sr else f"calibration fill of 1 GiB: writes {(fw or 0) / COPY_BYTES:.3f}x of the known bytes")
    er, ew = rec.get("ecopy_read"), rec.get("ecopy_write")
    if er:
        lines.append(f"calibration elementwise copy (1 GiB read + 1 GiB written): DRAM reads {er[0] / COPY_BYTES:.3f}x, "
                     f"all reads {er[1] / COPY_BYTES:.3f}x, writes {(ew or 0) / COPY_BYTES:.3f}x of the known bytes")
    lines.append(f"{'kernel':46s} {'dispatches':>10s} {'algorithmic MB':>15s} {'DRAM read MB':>13s} "
                 f"{'all read MB':>12s} {'write MB':>9s} {'read/alg':>9s}")
    for k in rec["kernels"]:
        lines.append(f"{k['kernel'][:46]:46s} {k['dispatches']:10d} {k['algorithmic_bytes'] / 1e6:15.1f} "
                     f"{k['read_dram_bytes'] / 1e6:13.1f} {k['read_all_bytes'] / 1e6:12.1f} "
                     f"{(k['write_bytes'] or 0) / 1e6:9.2f} {k['read_ratio']:9.3f}")
    return "\n".join(lines)


MFMA_PEAK_BF16 = 2.5e15  # dense bf16 matrix-core peak of one MI355X, flop/s


def mfma(d: str) -> str:
    """Matrix-core use per kernel and grid, from one counter pass with the
    derived counters MfmaUtil (busy share of all SIMDs' matrix cores, %) and
    MfmaFlopsBF16, over the dispatches after the first k_entry (the cycles;
    prefill and the reference decode come before it)."""
    per = {}
    for r in _counter_rows(d):
        e = per.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"], "grid": r["Grid_Size"],
                                                   "t": (int(r["Start_Timestamp"]), int(r["End_Timestamp"]))})
        e[r["Counter_Name"]] = float(r["Counter_Value"])
    ids = sorted(per)
    first = next((i for i in ids if "k_entry" in per[i]["name"]), None)
    if first is None:
        raise ValueError("no k_entry dispatch: run with k_entry in the kernel filter")
    agg = {}
    for i in ids:
        e = per[i]
        if i < first or "k_entry" in e["name"]:
            continue
        a = agg.setdefault((_short(e["name"]), e["grid"]), [0, 0.0, 0.0, 0.0])
        a[0] += 1
        a[1] += e.get("MfmaUtil", 0.0)
        a[2] += e.get("MfmaFlopsBF16", 0.0)
        a[3] += (e["t"][1] - e["t"][0]) * 1e-9
    out = [f"{'kernel':30s} {'grid':>8s} {'calls':>6s} {'MFMA util %':>11s} {'GFLOP/call':>10s} "
           f"{'us/call':>8s} {'TFLOP/s':>8s} {'of peak':>8s}"]
    for (name, grid), (n, u, f, t) in sorted(agg.items(), key=lambda kv: -kv[1][3]):
        rate = f / t if t > 0 else 0.0
        out.append(f"{name[:30]:30s} {grid:>8s} {n:6d} {u / n:11.2f} {f / n / 1e9:10.3f} {t / n * 1e6:8.2f} "
                   f"{rate / 1e12:8.1f} {rate / MFMA_PEAK_BF16:8.4f}")
    return "\n".join(out)


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    a = sub.add_parser("stats")
    a.add_argument("csv")
    a.add_argument("--cmd", default="")
    t = sub.add_parser("timeline")
    t.add_argument("csv")
    t.add_argument("--cycles", type=int, required=True)
    t.add_argument("--skip", type=int, default=0)
    t.add_argument("--cmd", default="")
    gp = sub.add_parser("gaps")
    gp.add_argument("csv")
    gp.add_argument("--cycles", type=int, required=True)
    gp.add_argument("--skip", type=int, default=0)
    gp.add_argument("--cmd", default="")
    b = sub.add_parser("traffic")
    b.add_argument("read_dir")
    b.add_argument("write_dir")
    b.add_argument("schedule")
    b.add_argument("--cmd", default="")
    b.add_argument("--write-json", action="store_true")
    mf = sub.add_parser("mfma")
    mf.add_argument("dir")
    mf.add_argument("--cmd", default="")
    args = ap.parse_args(argv)
    if args.what == "stats":
        if args.cmd:
            print(f"command: {args.cmd}")
        print(stats(args.csv))
    elif args.what == "timeline":
        if args.cmd:
            print(f"command: {args.cmd}")
        print(timeline(args.csv, args.cycles, args.skip))
    elif args.what == "gaps":
        if args.cmd:
            print(f"command: {args.cmd}")
        print(gaps(args.csv, args.cycles, args.skip))
    elif args.what == "mfma":
        if args.cmd:
            print(f"command: {args.cmd}")
        print(mfma(args.dir))
    else:
        rec = traffic(args.read_dir, args.write_dir, args.schedule)
        rec["command"] = args.cmd
        print(traffic_table(rec))
        if args.write_json:
            json.dump(rec, open(TRAFFIC_JSON, "w"), indent=2)


if __name__ == "__main__":
    sys.exit(main())
