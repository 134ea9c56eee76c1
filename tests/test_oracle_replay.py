"""Pins of the integer replay of the SPD schedule (CPU only).

Fed only the integers that floating point decided in a full oracle run (the
draft module's prediction, the target token and, under sampling, the accept
bit), the replay must reproduce every other integer of every cycle of that
run: position, occupancy, pending row, draft after the policy, exit, accept
decision, all KV lengths, the draft module's committed length and the emitted
count.  The full state machine it is compared with is itself pinned by
losslessness and the closed forms (test_oracle_spd.py).
"""
import pytest

import seeded_inputs as si
from oracle import SPDOracle, ar_greedy
from oracle.replay import Replay, ReplayError
from tests.test_oracle_spd import MODELS, _policies, _setup

FIELDS = ["t", "a", "pending_row", "draft", "exit_pos", "y", "accept", "kv_len", "pdm_len", "emitted"]


def _replay(w, first, logs, policy, sample=False):
    r = Replay(w.n, w.L, w.P, first, policy=policy, sample=sample, post=w.schedule == "post", split=w.split)
    out = []
    for l in logs:
        ex = l["exit_pos"] >= 0
        out.append(r.step(l["pdm_raw"], l["y"] if ex else None, l["accept"] if ex else None))
    return out


def _same(logs, rep):
    assert len(logs) == len(rep)
    for l, q in zip(logs, rep):
        for f in FIELDS:
            assert l[f] == q[f], (l["cycle"], f, l[f], q[f])


@pytest.mark.parametrize("sched", ["pre", "post"])
@pytest.mark.parametrize("mi", range(len(MODELS)))
def test_replay_reproduces_greedy_runs(mi, sched):
    if sched == "post" and MODELS[mi]["n"] < 2:
        pytest.skip("the post-step schedule needs two stages")
    w, W, prompt, u = _setup(G=14, schedule=sched, **MODELS[mi])
    ref, _ = ar_greedy(w, W, prompt, w.G)
    for name, pol in _policies(w, ref, u).items():
        o = SPDOracle(w, W, policy=pol, uniforms=u)
        toks, logs = o.run(prompt, w.G)
        _same(logs, _replay(w, toks[w.P], logs, pol))


@pytest.mark.parametrize("mi,temp,sched", [(0, 1.0, "pre"), (3, 0.1, "pre"), (5, 0.1, "pre"), (0, 1.0, "post"),
                                           (5, 0.1, "post")])
def test_replay_reproduces_sampling_runs(mi, temp, sched):
    w, W, prompt, u = _setup(G=14, mode="sample", temperature=temp, schedule=sched, **MODELS[mi])
    o = SPDOracle(w, W, uniforms=u)
    toks, logs = o.run(prompt, w.G)
    assert any(l["accept"] == 1 for l in logs) and any(l["accept"] == 0 for l in logs)
    _same(logs, _replay(w, toks[w.P], logs, None, sample=True))


def test_replay_tracks_tokens_in_flight_and_drafting_cycle():
    w, W, prompt, u = _setup(G=14, **MODELS[2])
    ref, _ = ar_greedy(w, W, prompt, w.G)
    pol = _policies(w, ref, u)["p0.8"]
    o = SPDOracle(w, W, policy=pol, uniforms=u)
    toks, logs = o.run(prompt, w.G)
    rep = _replay(w, toks[w.P], logs, pol)
    for q in rep:
        # in-flight positions are the newest a positions, the newest one last
        pos = [p for p, _ in q["inflight_tokens"]]
        assert pos == list(range(q["t"] - q["a"] + 1, q["t"] + 1))
        if q["exit_pos"] >= 0:
            # the draft of the verified position came from the cycle that had the exiting token newest
            assert rep[q["drafted_at"]]["t"] == q["exit_pos"]
            assert rep[q["drafted_at"]]["draft"] == logs[q["drafted_at"]]["draft"]


def test_replay_rejects_inconsistent_input():
    w, W, prompt, u = _setup(G=10, **MODELS[0])
    o = SPDOracle(w, W, uniforms=u)
    toks, logs = o.run(prompt, w.G)
    r = Replay(w.n, w.L, w.P, toks[w.P])
    with pytest.raises(ReplayError):
        for l in logs:
            r.step(l["pdm_raw"])          # exits without a target token
