"""Benchmark: SPD cycles/s and accepted tokens/s on one MI355X.

A step is one complete SPD generation from the post-prefill state of the
workload (all cycles until G tokens are emitted) -- every row of the cycle
(entry, stage-grouped decode, split-KV attention, anchor taps, verification,
rollback, draft-module FC + layers + head, two-stream overlap) runs in it.
Between steps the engine is rolled back to the prompt (spd_rollback), which
restores the post-prefill state exactly; the steps are therefore identical.

Workload (default): the 4B-class target (L=32, d=2560, 20/4 heads x 128,
SwiGLU 9728, V=151936) split into n=8 stages, draft module Ls=4, anchors
[0,8,16,24,31], random-init bf16 weights, 512-token random prompt, 256
greedy tokens, seeded forced acceptance 0.8.

Besides `value` (cycles/s) the line reports tokens/s, the fraction of HBM
peak per cycle from the algorithmic bytes, the draft bubble, the roofline of
the dominant kernel (stage-grouped gate/up projection, timed with HIP events
on its own stream inside the timed region) and the CPU oracle timed on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM = 8.0e12  # MI355X HBM3E, bytes/s


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def stage_ranges(w):
    """Layers of each stage: L/n each, or the workload's non-uniform split."""
    sizes = list(w.split) if getattr(w, "split", ()) else [w.L // w.n] * w.n
    starts = [sum(sizes[:k]) for k in range(w.n + 1)]
    return [range(starts[k], starts[k + 1]) for k in range(w.n)]


def cycle_bytes(w, rec, es):
    """Algorithmic HBM bytes of one executed cycle (weights + KV reads)."""
    L, d, F, V, n = w.L, w.d, w.F, w.V, w.n
    stages = stage_ranges(w)
    qkv = (w.Hq + 2 * w.Hkv) * w.hd
    W_layer = (qkv * d + d * w.Hq * w.hd + 2 * F * d + d * F) * es
    kv_pos = 2 * w.Hkv * w.hd * es
    P_attn = getattr(w, "attn_period", 0)
    lin_state = 2 * w.Hkv * (w.hd * w.hd + w.hd) * 4  # a linear layer reads and writes its fp32 state
    t, a = int(rec["t"]), int(rec["occupancy"])
    # a draft tree's stage groups stream their weights once for all their
    # nodes; each node reads its own KV (nodes per stage taken as the mean)
    per_stage = (int(rec["nodes"]) / a) if getattr(w, "width", 1) > 1 and a > 0 else 1.0
    b = sum(len(stages[k]) for k in range(a)) * W_layer
    for k in range(a):
        for l in stages[k]:
            linear = P_attn > 0 and l % P_attn != P_attn - 1
            b += lin_state if linear else per_stage * (t - k + 1) * kv_pos
    if rec["exit_pos"] >= 0:
        b += V * d * es
    # draft module: FC patterns present, Ls layers, head, KV reads
    def pattern(k):  # last anchor b_i <= lmax(k), the layers of the first k stages
        lm = stages[k].start if k < n else L
        return max(i for i, bb in enumerate(w.anchors) if bb <= lm)
    if getattr(w, "schedule", "pre") == "post":
        pats = {pattern(k) for k in range(1, a + 1)}  # rows at depths a .. 1
    else:
        pats = {pattern(k) for k in range(a)}
        if rec["pending_row"]:
            pats.add(pattern(n))
    b += sum((f + 1) * d * d * es for f in pats)
    b += w.Ls * W_layer + V * d * es
    b += w.Ls * (t + 1) * kv_pos
    return b


def traffic_bytes(workload):
    """HBM bytes per gate/up launch from the committed counter summary, or
    None if it was taken on another workload or the kernel sources changed
    since the counters were taken."""
    from pipelined_draft_verify_amd import profile_summary as ps
    try:
        rec = json.load(open(ps.TRAFFIC_JSON))
    except (OSError, ValueError):
        return None
    if rec.get("workload") != workload or rec.get("source_hash") != ps.kernel_source_hash():
        return None
    return int(rec["traffic_bytes_per_launch"])


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="4b_n8")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-cycles", type=int, default=192)
    ap.add_argument("--eager", action="store_true",
                    help="launch every kernel from the host in the timed region (no HIP graphs)")
    ap.add_argument("--serialized", action="store_true",
                    help="run the draft module on the stage stream ahead of the stage step (no overlap)")
    ap.add_argument("--schedule", choices=["pre", "post"], default="pre",
                    help="draft-module features before (pre) or after (post) the stage step")
    ap.add_argument("--dump-schedule", default="",
                    help="write the step's per-cycle schedule (occupancy, exit) to this json file")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU; --gpus must be 1"}))
        sys.exit(2)

    import torch
    import seeded_inputs as si
    from pipelined_draft_verify_amd import SPDEngine

    w = si.workload(args.workload)
    if args.schedule != "pre":
        w = w.replace(schedule=args.schedule)
    es = 2 if w.dtype == "bf16" else 4
    t0 = time.time()
    T = si.make_weights(w, "cuda:0")
    torch.cuda.synchronize()
    log(f"weights generated on GPU in {time.time() - t0:.1f}s")
    # dispatches of known HBM traffic that the traffic counters are checked
    # on: a 1 GiB fill (writes), a sum over it (reads) and an elementwise
    # 1 GiB copy (x * 1: reads and writes), issued last before the engine
    calib_src = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")
    calib_sum = calib_src.sum()
    calib_dst = torch.empty_like(calib_src)
    torch.mul(calib_src, 1.0, out=calib_dst)
    torch.cuda.synchronize()
    assert float(calib_sum) == float(1 << 28)
    del calib_src, calib_dst, calib_sum
    eng = SPDEngine(w, T)
    uni = si.make_uniforms(w)
    eng.set_uniforms(uni)
    prompt = si.make_prompt(w)
    t0 = time.time()
    first = eng.prefill(prompt)
    log(f"prefill {w.P} tokens in {time.time() - t0:.2f}s")
    if w.policy == "forced":
        t0 = time.time()
        ar = eng.generate_ar(w.G - 1)
        log(f"reference AR decode of {w.G - 1} tokens in {time.time() - t0:.2f}s")
        eng.rollback(w.P, first)
        if getattr(w, "width", 1) > 1:
            eng.set_tree_forced(list(prompt) + [first] + ar, w.p_accept, w.p_tree)
        else:
            eng.set_forced(list(prompt) + [first] + ar, w.p_accept)

    # discover the step's cycle count (deterministic) with a logged run
    recs = eng.run(batch=128)
    K_c = len(recs)
    acc = recs[recs["exit_pos"] >= 0]
    log(f"one step = {K_c} cycles; {int((acc['accepted'] == 1).sum())}/{len(acc)} verifications accepted")
    if args.dump_schedule:
        json.dump({"workload": w.name, "cycles": [{"t": int(r["t"]), "occupancy": int(r["occupancy"]),
                                                    "exit_pos": int(r["exit_pos"]), "nodes": int(r["nodes"])}
                                                   for r in recs]}, open(args.dump_schedule, "w"))

    def step(log_buf=False):
        eng.rollback(w.P, first)
        return eng.enqueue(K_c, log=log_buf)

    for _ in range(args.warmup):
        step()
        eng.sync()

    # timed region: graph launch mode, per-cycle HIP events for cycle times / bubble
    eng.set_launch_mode(not args.eager, args.serialized)
    torch.cuda.synchronize()
    eng.timing(True)
    cyc_times = []
    enq_s = 0.0
    t_start = time.perf_counter()
    for _ in range(args.steps):
        eng.rollback(w.P, first)
        t_e = time.perf_counter()
        eng.enqueue(K_c, log=False)
        enq_s += time.perf_counter() - t_e
        eng.sync()
        n_c, cyc, _, _ = eng.timing_read(K_c)
        cyc_times.extend(cyc)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    eng.timing(False)
    log(f"timed: {elapsed / args.steps * 1e3:.1f} ms/step, host enqueue {enq_s / args.steps * 1e3:.1f} ms/step")

    # dominant-kernel timing: one more step, each gate/up launch bracketed by
    # HIP events on the stage stream (eager launch mode)
    eng.set_launch_mode(False, args.serialized)
    eng.timing(True)
    eng.rollback(w.P, first)
    t_e = time.perf_counter()
    eng.enqueue(K_c, log=False)
    eng.sync()
    eager_s = time.perf_counter() - t_e
    _, _, gu_ms, gu_n = eng.timing_read(K_c)
    eng.timing(False)
    eng.set_launch_mode(not args.eager, args.serialized)
    log(f"eager instrumented step: {eager_s * 1e3:.1f} ms")
    cycles = args.steps * K_c
    value = cycles / elapsed
    tokens_per_s = args.steps * (w.G - 1) / elapsed
    # per-cycle algorithmic bytes and timing
    per_cycle_bytes = np.array([cycle_bytes(w, r, es) for r in recs], dtype=np.float64)
    cyc_arr = np.array(cyc_times, dtype=np.float64).reshape(-1, 3)  # stage end, pdm end, cycle end (ms)
    reps = len(cyc_arr) // K_c
    cyc_end = cyc_arr[:, 2].reshape(reps, K_c).mean(axis=0)
    bubble = float(np.maximum(0.0, cyc_arr[:, 1] - cyc_arr[:, 0]).sum() / cyc_arr[:, 2].sum())
    hbm_frac = float(per_cycle_bytes.sum() / (cyc_end.sum() * 1e-3) / PEAK_HBM)
    hbm_frac_wall = float(per_cycle_bytes.sum() * args.steps / elapsed / PEAK_HBM)
    per_cycle_frac = per_cycle_bytes / (cyc_end * 1e-3) / PEAK_HBM
    occ = recs["occupancy"]
    full = occ == w.n
    # where the time and the bubble go, by occupancy (stderr diagnostics)
    st = cyc_arr[:, 0].reshape(reps, K_c).mean(axis=0)
    pd = cyc_arr[:, 1].reshape(reps, K_c).mean(axis=0)
    for a in sorted(set(int(x) for x in occ)):
        sel = occ == a
        log(f"occupancy {a}: {int(sel.sum())} cycles, stage {st[sel].mean() * 1e3:.0f} us, "
            f"draft {pd[sel].mean() * 1e3:.0f} us, cycle {cyc_end[sel].mean() * 1e3:.0f} us, "
            f"share of the bubble {np.maximum(0, pd[sel] - st[sel]).sum() / cyc_end.sum():.4f}")
    hbm_full = float(per_cycle_bytes[full].sum() / (cyc_end[full].sum() * 1e-3) / PEAK_HBM) if full.any() else None
    # dominant kernel: stage gate/up GEMV; algorithmic bytes = a * 2F * d * es per launch
    stages = stage_ranges(w)
    gu_bytes_step = float(sum(sum(len(stages[k]) for k in range(int(r["occupancy"]))) for r in recs)
                          * 2 * w.F * w.d * es)
    gu_launches_step = K_c * max(len(r) for r in stages)  # one launch per sub-step
    assert gu_n == gu_launches_step, (gu_n, gu_launches_step)
    gu_avg_s = gu_ms * 1e-3 / gu_n
    gu_bytes_launch = gu_bytes_step / gu_launches_step
    achieved = gu_bytes_launch / gu_avg_s

    out = {
        "metric": "SPD cycles/s and accepted tokens/s at 1 GPU; % of peak HBM GB/s per cycle",
        "value": round(value, 3),
        "unit": "cycles/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded random-init weights and prompt)",
        "config": {
            "workload": f"{w.name}: L={w.L} d={w.d} heads {w.Hq}/{w.Hkv}x{w.hd} FFN {w.F} V={w.V} n={w.n} "
                        f"Ls={w.Ls} anchors={w.anchors} prompt {w.P} gen {w.G} "
                        f"{w.mode}{' top-k ' + str(w.top_k) if w.top_k else ''} "
                        f"{w.policy}{' p=' + str(w.p_accept) if w.policy == 'forced' else ''}"
                        f"{' draft tree W=' + str(w.width) + ' p_tree=' + str(w.p_tree) if w.width > 1 else ''}"
                        f" {w.schedule}-step drafting",
            "cycles_per_step": K_c,
            "parallelism": "single GPU, " + ("one stream (draft module serialized)" if args.serialized
                                             else "two HIP streams"),
            "launch": "eager" if args.eager else "hip graphs",
        },
        "tokens_per_s": round(tokens_per_s, 3),
        "hbm_frac_per_cycle": round(hbm_frac, 4),
        "hbm_frac_wall_clock": round(hbm_frac_wall, 4),
        "hbm_frac_full_cycles": round(hbm_full, 4) if hbm_full is not None else None,
        "hbm_frac_cycle_median": round(float(np.median(per_cycle_frac)), 4),
        "hbm_frac_cycle_p10": round(float(np.percentile(per_cycle_frac, 10)), 4),
        "tokens_per_cycle": round((w.G - 1) / K_c, 4),
        "L_acc": round((w.G - 1) / K_c * w.n, 4),
        "bubble_frac": round(bubble, 4),
        "accepted_verifications": int((acc["accepted"] == 1).sum()),
        "verifications": int(len(acc)),
        "roofline": {
            "bound": "hbm",
            "kernel": "k_gemv_stage<bf16,SWIGLU> (stage-grouped gate/up projection)",
            "achieved": round(achieved / 1e9, 1),
            "peak": PEAK_HBM / 1e9,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM, 4),
            "traffic": traffic_bytes(w.name),
            "avg_launch_us": round(gu_avg_s * 1e6, 2),
            "bytes_per_launch": int(gu_bytes_launch),
            "timed_over": "every gate/up launch of one eager-launched step of the workload",
        },
    }

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, T, prompt, uni, args.cpu_cycles)
    eng.close()
    print(json.dumps(out), flush=True)


def cpu_baseline(w, T, prompt, uni, n_cycles):
    """The oracle timed on this host over a bounded sample of the workload."""
    import torch
    import seeded_inputs as si
    from oracle import ForcedPolicy, SPDOracle
    from oracle.spd import ar_continue
    from oracle.tree import TreeForcedPolicy, TreeSPDOracle

    t0 = time.time()
    W = si.nest_weights(si.weights_numpy_f32(T), w)
    log(f"cpu baseline: host fp32 weights in {time.time() - t0:.1f}s")
    t0 = time.time()
    pol = None
    tree = getattr(w, "width", 1) > 1
    o = TreeSPDOracle(w, W, w.width) if tree else SPDOracle(w, W, uniforms=uni)
    o.prefill(prompt, matrix=True)
    if w.policy == "forced":
        ref = ar_continue(o, n_cycles + w.n)
        pol = TreeForcedPolicy(ref, w.p_accept, w.p_tree, uni, w.V) if tree else ForcedPolicy(ref, w.p_accept, uni, w.V)
        o.policy = pol
    log(f"cpu baseline: oracle prefill{' + reference decode' if pol else ''} in {time.time() - t0:.1f}s")
    t0 = time.perf_counter()
    for _ in range(n_cycles):
        o.cycle()
    dt = time.perf_counter() - t0
    threads = _blas_threads()
    return {"value": round(n_cycles / dt, 4), "unit": "cycles/s", "cores": threads, "kind": "oracle",
            "host_cpus": os.cpu_count(),
            "sample": f"first {n_cycles} SPD cycles after the {w.P}-token prefill of the same workload "
                      f"(numpy fp32, {threads} BLAS threads of {os.cpu_count()} host CPUs visible); "
                      f"{dt:.1f}s of CPU work"}


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if info:
            return int(info[0]["num_threads"])
    except Exception:
        pass
    return os.cpu_count()


if __name__ == "__main__":
    main()
