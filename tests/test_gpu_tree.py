"""GPU parity of draft trees (draft_width W >= 2) against the tree oracle.

[RB] prerequisites ("draft tree") and [PL] appendix B (width-4 trees in
SPD); the reading is oracle/tree.py's.  The HIP path and the oracle run the
same seeded weights, prompt, uniforms and forced tree policy.  Every cycle's
integers must agree: the newest position, the occupancy, the nodes in
flight, the entered nodes (parent rank and token, in rank order), the
committed-row flag, the exit, the target token, the accept decision and the
kept child's rank, the committed KV length (every layer), the draft module's
committed length and the emitted count.  Where floating point decides (the
target's argmax, the ranking of the candidates), a differing GPU choice is a
near-tie only if it is within the argmax tolerance (1e-4 fp32, 0.05 bf16) in
the oracle's own logits or scores; the oracle then follows it.
"""
import numpy as np
import pytest

import seeded_inputs as si
from oracle import ar_greedy
from oracle.tree import TreeForcedPolicy, TreeSPDOracle
from tests.gpu_common import gpu_workload_tiny

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 0.05}

VARIANTS = {
    "f32_n2_w2": dict(dtype="f32", L=4, n=2, width=2, p1=0.3, pW=0.7, seed=91),
    "f32_n4_w3": dict(dtype="f32", L=4, n=4, anchors=[0, 1, 2, 3, 4], width=3, p1=0.3, pW=0.8, G=30, seed=92),
    "f32_n4_w4_tree_only": dict(dtype="f32", L=4, n=4, anchors=[0, 1, 2, 3, 4], width=4, p1=0.0, pW=0.8, G=30,
                                seed=93),
    "bf16_n4_w4_gqa": dict(dtype="bf16", L=8, n=4, Hq=8, Hkv=2, F=768, V=500, anchors=[0, 2, 4, 8], Ls=2,
                           width=4, p1=0.3, pW=0.8, G=30, seed=94),
    "bf16_n8_w3": dict(dtype="bf16", L=8, n=8, Ls=1, anchors=[0, 3, 8], width=3, p1=0.5, pW=0.8, G=30, seed=95),
    "bf16_hd128_w2": dict(dtype="bf16", Hq=2, Hkv=1, hd=128, F=512, V=700, width=2, p1=0.4, pW=0.9, G=24,
                          seed=96, norm_gain="random"),
    "f32_natural_w4": dict(dtype="f32", L=4, n=2, width=4, p1=None, pW=None, G=16, seed=97),
}


def _gpu(w, T, prompt, uni, ref, p1, pW):
    from pipelined_draft_verify_amd import SPDEngine

    eng = SPDEngine(w, {k: v.to("cuda:0") for k, v in T.items()})
    eng.set_uniforms(uni)
    if p1 is not None:
        eng.set_tree_forced(ref, p1, pW)
    first = eng.prefill(prompt)
    recs = eng.run(batch=64)
    toks = eng.tokens(0, w.P + w.G)
    eng.close()
    return first, recs, toks


def _teacher(recs, first):
    t = {("first", 0): int(first)}
    for r in recs:
        c = int(r["cycle"])
        if r["exit_pos"] >= 0:
            t[("y", c)] = int(r["target_token"])
        if r["n_new"] > 0 and r["new_parent"][0] >= 0:
            t[("entry", c)] = [(int(r["new_parent"][k]), int(r["new_token"][k])) for k in range(int(r["n_new"]))]
    return t


def run_and_compare(w, T, W, prompt, uni, ref, p1, pW):
    first, recs, toks = _gpu(w, T, prompt, uni, ref, p1, pW)
    pol = None if p1 is None else TreeForcedPolicy(ref, p1, pW, uni, w.V)
    o = TreeSPDOracle(w, W, w.width, policy=pol, teacher=_teacher(recs, first), tol=TOL[w.dtype])
    otoks, ologs = o.run(prompt, w.G)
    assert not o.mismatch, o.mismatch[:5]
    assert toks == otoks
    assert len(recs) == len(ologs), (len(recs), len(ologs))
    for r, l in zip(recs, ologs):
        c = int(r["cycle"])
        got = (int(r["t"]), int(r["occupancy"]), int(r["nodes"]), int(r["n_new"]), int(r["pending_row"]),
               int(r["exit_pos"]), int(r["target_token"]), int(r["accepted"]), int(r["accepted_rank"]),
               int(r["pdm_len"]), int(r["emitted"]))
        want = (l["t"], l["a"], l["nodes"], l["n_new"], l["pending_row"], l["exit_pos"], l["y"], l["accept"],
                l["acc_rank"], l["pdm_len"], l["emitted"])
        assert got == want, (c, got, want)
        assert [int(x) for x in r["new_parent"][: l["n_new"]]] == l["new_parent"], c
        assert [int(x) for x in r["new_token"][: l["n_new"]]] == l["new_token"], c
        assert all(int(x) == l["committed"] for x in r["kv_len"][: w.L]), (c, "committed KV length")
        assert int(r["flags"]) == 0, (c, int(r["flags"]))
    return recs, ologs, o


@pytest.mark.parametrize("name", sorted(VARIANTS))
def test_tree_matches_oracle(name):
    kw = dict(VARIANTS[name])
    p1, pW = kw.pop("p1"), kw.pop("pW")
    w = gpu_workload_tiny(**kw)
    T = si.make_weights(w, "cpu")
    W = si.nest_weights(si.weights_numpy_f32(T), w)
    prompt = si.make_prompt(w)
    uni = si.make_uniforms(w)
    ref, _ = ar_greedy(w, W, prompt, w.G)
    recs, ologs, o = run_and_compare(w, T, W, prompt, uni, ref, p1, pW)
    print(name, "adopted", o.adopted[:5], "cycles", len(recs))
    assert len(o.adopted) <= 3, o.adopted
    widths = recs["n_new"]
    assert widths.max() == w.width  # the tree widens
    if p1 is not None:
        ex = recs[recs["exit_pos"] >= 0]
        assert (ex["accepted"] == 1).any() and (ex["accepted"] == 0).any()
    if name == "f32_n4_w4_tree_only":
        # p1 = 0: the true token is never the best-ranked candidate, which a
        # chain would never accept; the tree keeps it, often not as the first child
        acc = recs[(recs["exit_pos"] >= 0) & (recs["accepted"] == 1)]
        assert len(acc) > 0 and (acc["accepted_rank"] > 0).any()


def test_tree_graph_and_eager_agree_and_rollback_restarts():
    """Graph-replayed and host-launched tree cycles give identical records;
    a host rollback to the prompt restarts the same generation."""
    from pipelined_draft_verify_amd import SPDEngine

    w = gpu_workload_tiny(dtype="bf16", L=8, n=4, anchors=[0, 2, 4, 8], Ls=2, width=3, G=30, seed=98)
    T = si.make_weights(w, "cpu")
    W = si.nest_weights(si.weights_numpy_f32(T), w)
    prompt = si.make_prompt(w)
    uni = si.make_uniforms(w)
    ref, _ = ar_greedy(w, W, prompt, w.G)
    eng = SPDEngine(w, {k: v.to("cuda:0") for k, v in T.items()})
    eng.set_uniforms(uni)
    eng.set_tree_forced(ref, 0.3, 0.8)
    first = eng.prefill(prompt)
    out = []
    for mode in (True, False, True):
        eng.rollback(w.P, first)
        eng.set_launch_mode(mode)
        recs = eng.run(batch=16)
        recs["cycle"] -= recs["cycle"][0]
        out.append((recs.tobytes(), eng.tokens(0, w.P + w.G)))
    eng.close()
    assert out[0] == out[1] == out[2]
