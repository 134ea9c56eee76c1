"""Full-size draft tree: the 4B-class n=8 workload with width-4 trees.

[RB] prerequisites ("draft tree"), [PL] appendix B; the reading is
oracle/tree.py's.  The generation runs on the GPU exactly as the benchmark
times it (device-generated weights, graph launch, forced tree policy from the
GPU's own autoregressive decode).  The tree oracle is too slow to follow a
full-size run cycle by cycle, so the run is checked by what holds at any
size:

  * every cycle record obeys the tree's invariants: occupancy in 1..n, at
    most 1 + (a - 1) W nodes in flight, 1..W entered nodes (one after a
    re-seed), every layer's committed KV length equal, an accepted child's
    rank below W, no device flags;
  * the cycle count obeys the chain's closed form K = n + (G - 2) + (n - 1) R
    (a rejection still costs n - 1 refill cycles), every position from the
    prompt's end is verified once, in order;
  * losslessness: the output is the target's own greedy continuation;
  * every verification: the target token of each exit against the oracle's
    forward over the final sequence (a differing choice must be a near-tie);
  * the verification logits of the last exit against the oracle's (rel-L2).
"""
import gc

import numpy as np
import pytest

import seeded_inputs as si
from oracle import schedule
from tests import full_size as fs

pytestmark = pytest.mark.gpu

NAME = "4b_tree4_n8"
_C = {}


def _run():
    if "run" in _C:
        return _C["run"]
    import torch
    from pipelined_draft_verify_amd import SPDEngine

    w = si.workload(NAME)
    T = si.make_weights(w, "cuda:0")
    eng = SPDEngine(w, T)
    eng.set_launch_mode(True)
    uni = si.make_uniforms(w)
    eng.set_uniforms(uni)
    prompt = si.make_prompt(w)
    first = int(eng.prefill(prompt))
    ar = eng.generate_ar(w.G - 1)
    ref = [int(x) for x in prompt] + [first] + [int(x) for x in ar]
    eng.rollback(w.P, first)
    eng.set_tree_forced(ref, w.p_accept, w.p_tree)
    recs = eng.run(batch=256)
    toks = [int(x) for x in eng.tokens(0, w.P + w.G)]
    last_logits = eng.logits()
    eng.close()
    del eng
    flat = si.weights_numpy_f32(T)
    del T
    gc.collect()
    torch.cuda.empty_cache()
    _C["run"] = dict(w=w, W=si.nest_weights(flat, w), prompt=prompt, uni=uni, first=first, ref=ref, recs=recs,
                     toks=toks, last_logits=last_logits)
    return _C["run"]


def test_tree_full_size_integers_and_losslessness():
    run = _run()
    w, recs = run["w"], run["recs"]
    n, W = w.n, w.width
    assert W == 4
    for i, r in enumerate(recs):
        a = int(r["occupancy"])
        assert 1 <= a <= n, (i, a)
        assert 1 <= int(r["nodes"]) <= 1 + (a - 1) * W, (i, int(r["nodes"]), a)
        nn = int(r["n_new"])
        assert 1 <= nn <= W, (i, nn)
        if int(r["new_parent"][0]) < 0:
            assert nn == 1, (i, "a re-seed enters one node")
        kv = [int(x) for x in r["kv_len"][: w.L]]
        assert len(set(kv)) == 1, (i, "committed length differs between layers")
        if int(r["exit_pos"]) >= 0:
            assert kv[0] == int(r["exit_pos"]) + 1, (i, kv[0], int(r["exit_pos"]))
            acc = int(r["accepted"])
            assert acc in (0, 1)
            assert (int(r["accepted_rank"]) in range(W)) if acc else int(r["accepted_rank"]) == -1, i
        assert int(r["flags"]) == 0, (i, int(r["flags"]))
    ex = recs[recs["exit_pos"] >= 0]
    R = int((ex["accepted"][: w.G - 2] == 0).sum())
    print(f"{NAME}: {len(recs)} cycles, {len(ex)} verifications, {R} rejections, "
          f"{int((ex['accepted_rank'] > 0).sum())} accepted at a rank > 0")
    assert len(ex) == w.G - 1
    assert list(ex["exit_pos"]) == list(range(w.P, w.P + w.G - 1))
    assert len(recs) == schedule.cycle_count(n, w.G, R)
    # the output: the first token, then each exit's target token; lossless
    assert run["toks"][w.P:w.P + w.G] == [run["first"]] + [int(x) for x in ex["target_token"]]
    assert run["toks"][w.P:w.P + w.G] == run["ref"][w.P:w.P + w.G]
    # the tree keeps true tokens the first rank missed
    assert (ex["accepted_rank"] > 0).any()


def test_tree_full_size_verifications_and_logits():
    run = _run()
    w, recs = run["w"], run["recs"]
    view = fs.OracleView(run)
    dec = fs.check_verifications(run, view, None)
    worst = max((a[3] for a in dec.adopted), default=0.0)
    print(f"{NAME} target tokens: {w.G} checked, {len(dec.adopted)} near-ties adopted (largest gap {worst:.3g})")
    assert not dec.mismatch, dec.mismatch[:5]
    assert len(dec.adopted) <= max(2, w.G // 50), dec.adopted[:10]
    j = int(recs[recs["exit_pos"] >= 0]["exit_pos"][-1])
    err = fs.rel_l2(run["last_logits"], view.logits_at(j))
    print(f"{NAME} last verification logits rel-L2 {err:.3g}")
    assert err <= fs.RTOL[w.dtype]
