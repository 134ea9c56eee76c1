"""Summaries of rocprofv3 output for the committed profiles/ files.

  python -m pipelined_draft_verify_amd.profile_summary stats <kernel_stats.csv> [--cmd "..."]
  python -m pipelined_draft_verify_amd.profile_summary traffic <fetch_dir> <write_dir> --cmd "..."

`traffic` reads two counter-collection runs (FETCH_SIZE, then WRITE_SIZE, KiB
per dispatch), scales each by what the same counter read for a plain copy of
known size (1 GiB read + 1 GiB written) and prints the HBM bytes per launch of
the stage-grouped gate/up GEMV, with a hash of the kernel sources they were
taken on; bench.py reports the traffic only while that hash still matches.
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
GU_REGEX = r"k_gemv_stage<unsigned short, 2>"
COPY_REGEX = r"copy"
COPY_BYTES = 1 << 30


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in ("common.h", "gemv.h"):
        h.update(open(os.path.join(HERE, "csrc", name), "rb").read())
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


def copy_reading(d: str, counter: str):
    """Counter value of the 1 GiB calibration copy: by far the largest copy dispatch."""
    vals = counter_values(d, counter, COPY_REGEX)
    return max(vals) if vals else None


def traffic(fetch_dir: str, write_dir: str):
    f_gu, n_gu = counter_avg(fetch_dir, "FETCH_SIZE", GU_REGEX)
    f_cp = copy_reading(fetch_dir, "FETCH_SIZE")
    w_gu, m_gu = counter_avg(write_dir, "WRITE_SIZE", GU_REGEX)
    w_cp = copy_reading(write_dir, "WRITE_SIZE")
    fs = COPY_BYTES / (f_cp * 1024.0)
    ws = COPY_BYTES / (w_cp * 1024.0)
    rec = {
        "kernel": "k_gemv_stage<bf16,SWIGLU>",
        "workload": "4b_n8",
        "source_hash": kernel_source_hash(),
        "fetch_kib_per_dispatch": f_gu, "write_kib_per_dispatch": w_gu,
        "dispatches": [n_gu, m_gu],
        "copy_fetch_kib": f_cp, "copy_write_kib": w_cp, "fetch_scale": fs, "write_scale": ws,
        "traffic_bytes_per_launch": f_gu * 1024.0 * fs + w_gu * 1024.0 * ws,
    }
    return rec


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    a = sub.add_parser("stats")
    a.add_argument("csv")
    a.add_argument("--cmd", default="")
    b = sub.add_parser("traffic")
    b.add_argument("fetch_dir")
    b.add_argument("write_dir")
    b.add_argument("--cmd", default="")
    b.add_argument("--write-json", action="store_true")
    args = ap.parse_args(argv)
    if args.what == "stats":
        if args.cmd:
            print(f"command: {args.cmd}")
        print(stats(args.csv))
    else:
        rec = traffic(args.fetch_dir, args.write_dir)
        rec["command"] = args.cmd
        print(json.dumps(rec, indent=2))
        if args.write_json:
            json.dump(rec, open(TRAFFIC_JSON, "w"), indent=2)


if __name__ == "__main__":
    sys.exit(main())
