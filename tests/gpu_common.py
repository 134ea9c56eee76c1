"""Helpers shared by the GPU tests: run the HIP path and the oracle on the same
seeded inputs and compare them."""
from __future__ import annotations

import numpy as np

import seeded_inputs as si

INT_FIELDS = [("t", "t"), ("occupancy", "a"), ("pending_row", "pending_row"), ("pdm_argmax", "pdm_raw"),
              ("draft", "draft"), ("exit_pos", "exit_pos"), ("target_token", "y"), ("accepted", "accept"),
              ("pdm_len", "pdm_len"), ("emitted", "emitted")]


def gpu_workload_tiny(**kw):
    """A small model whose shapes the library accepts (d, F, Hq*hd multiples of 256)."""
    base = dict(name="gt", dtype="f32", L=4, d=256, Hq=4, Hkv=2, hd=64, F=512, V=300, n=2, Ls=1,
                anchors=[0, 2, 4], P=20, G=24, seed=31)
    base.update(kw)
    return si.Workload(**base)


def run_gpu(w, T_cpu, prompt, uni=None, ref=None, p_accept=None, batch=64, per_cycle_hook=None):
    import torch
    from pipelined_draft_verify_amd import SPDEngine

    eng = SPDEngine(w, {k: v.to("cuda:0") for k, v in T_cpu.items()})
    if uni is not None:
        eng.set_uniforms(uni)
    if ref is not None:
        eng.set_forced(ref, p_accept)
    first = eng.prefill(prompt)
    if per_cycle_hook is None:
        recs = eng.run(batch=batch)
    else:
        out = []
        while True:
            buf = eng.enqueue(1)
            st = eng.sync()
            r = eng.records_of(buf)
            if r["flags"][0] & 8:
                break
            out.append(r)
            per_cycle_hook(eng, r[0])
            if st.done:
                break
        recs = np.concatenate(out)
    toks = eng.tokens(0, w.P + w.G)
    return eng, first, recs, toks


def run_gpu_with_sets(w, T_cpu, prompt, uni):
    """A sampling run, one cycle at a time, that also reads the logits behind
    every top-k truncation the GPU made: the draft module's at every cycle,
    the target's at every exit and after prefill.  The kept sets are the top-k
    ids of those logits (ties to the lower id, as the kernels rank them)."""
    from oracle.sampling import top_k_ids

    sets = {}

    def hook(eng, r):
        c = int(r["cycle"])
        sets[("qset", c)] = top_k_ids(eng.pdm_logits(), w.top_k)
        if r["exit_pos"] >= 0:
            sets[("pset", c)] = top_k_ids(eng.logits(), w.top_k)

    import torch
    from pipelined_draft_verify_amd import SPDEngine

    eng = SPDEngine(w, {k: v.to("cuda:0") for k, v in T_cpu.items()})
    eng.set_uniforms(uni)
    first = eng.prefill(prompt)
    sets[("pset_first", 0)] = top_k_ids(eng.logits(), w.top_k)
    out = []
    while True:
        buf = eng.enqueue(1)
        st = eng.sync()
        r = eng.records_of(buf)
        if r["flags"][0] & 8:
            break
        out.append(r)
        hook(eng, r[0])
        if st.done:
            break
    recs = np.concatenate(out)
    toks = eng.tokens(0, w.P + w.G)
    return eng, first, recs, toks, sets


def teacher_of(recs, first, sets=None):
    """Decisions the GPU took, keyed as the oracle's Decisions expects (with
    `sets`: also the top-k kept sets behind them)."""
    t = dict(sets or {})
    t[("first", 0)] = int(first)
    for r in recs:
        c = int(r["cycle"])
        t[("pdm", c)] = int(r["pdm_argmax"])
        t[("draft", c)] = int(r["pdm_argmax"])
        if r["exit_pos"] >= 0:
            t[("y", c)] = int(r["target_token"])
            t[("accept", c)] = bool(r["accepted"])
            t[("resample", c)] = int(r["target_token"])
    return t


def compare_logs(recs, ologs, L):
    """Bit-exact comparison of every integer field of every cycle."""
    assert len(recs) == len(ologs), f"cycle counts differ: gpu {len(recs)} oracle {len(ologs)}"
    for r, l in zip(recs, ologs):
        for gf, of in INT_FIELDS:
            assert int(r[gf]) == int(l[of]), (int(r["cycle"]), gf, int(r[gf]), l[of])
        assert list(map(int, r["kv_len"][:L])) == list(l["kv_len"]), (int(r["cycle"]), "kv_len")
        assert int(r["flags"]) == 0, (int(r["cycle"]), "flags", int(r["flags"]))


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))
