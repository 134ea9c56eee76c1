"""Pins of the oracle's SPD state machine (CPU only).

* Losslessness, by brute force: for random tiny models and every kind of
  draft policy, the SPD output equals plain greedy autoregressive decoding of
  the target, and the KV caches hold the same entries.
* The cycle count obeys the closed form derived from the schedule.
* KV lengths obey the per-stage formula and the rollback length.
* The cached (incremental) draft module equals a full recompute over the
  whole feature sequence.
* Planted mistakes in the oracle (wrong truncation length, dropped feature
  commit) are caught by these checks.
"""
import numpy as np
import pytest

import seeded_inputs as si
from oracle import SPDOracle, ForcedPolicy, NaturalPolicy, ar_greedy, schedule
from oracle.model import PDM, Target
from oracle.spd import FixedPolicy

MODELS = [
    dict(L=4, n=2, Ls=1, anchors=[0, 2, 3], Hq=4, Hkv=2, seed=11),
    dict(L=4, n=4, Ls=1, anchors=[0, 1, 2, 4], Hq=2, Hkv=2, seed=12),
    dict(L=6, n=3, Ls=2, anchors=[0, 1, 4, 6], Hq=4, Hkv=1, seed=13),
    dict(L=8, n=4, Ls=2, anchors=[0, 2, 4, 6, 7], Hq=4, Hkv=4, seed=14, dtype="bf16"),
    dict(L=8, n=8, Ls=1, anchors=[0, 3, 8], Hq=6, Hkv=3, seed=15, norm_gain="random"),
    dict(L=6, n=2, Ls=3, anchors=[0, 5], Hq=2, Hkv=1, seed=16, dtype="bf16"),
    # one stage: every token exits in the cycle it enters (one token per cycle)
    dict(L=4, n=1, Ls=2, anchors=[0, 2, 4], Hq=2, Hkv=1, seed=17),
]


def _setup(**kw):
    w = si.tiny(**kw)
    W = si.nest_weights(si.weights_numpy_f32(si.make_weights(w)), w)
    return w, W, si.make_prompt(w), si.make_uniforms(w)


def _policies(w, ref, u):
    G = len(ref)
    rng = np.random.default_rng(w.seed)
    every3 = [(q % 3) != 0 for q in range(G)]
    return {
        "natural": NaturalPolicy(),
        "right": ForcedPolicy(ref, 1.0, u, w.V),
        "wrong": ForcedPolicy(ref, 0.0, u, w.V),
        "p0.3": ForcedPolicy(ref, 0.3, u, w.V),
        "p0.8": ForcedPolicy(ref, 0.8, u, w.V),
        "every3": FixedPolicy(ref, every3, w.V),
        "random": FixedPolicy(ref, list(rng.random(G) < 0.5), w.V),
    }


def _rejects_before_last(logs, G):
    ver = [l for l in logs if l["exit_pos"] >= 0]
    return sum(1 for l in ver[: G - 2] if not l["accept"])


@pytest.mark.parametrize("mi", range(len(MODELS)))
def test_lossless_against_autoregressive(mi):
    w, W, prompt, u = _setup(G=14, **MODELS[mi])
    ref, ar = ar_greedy(w, W, prompt, w.G)
    for name, pol in _policies(w, ref, u).items():
        o = SPDOracle(w, W, policy=pol, uniforms=u)
        toks, logs = o.run(prompt, w.G)
        assert toks == ref, name
        # the KV entries of every verified position equal the AR ones
        upto = len(ref) - 1  # AR never computes the last token's KV
        for l in range(w.L):
            m = min(upto, o.target.kv[l].length)
            assert np.array_equal(o.target.kv[l].K[:m], ar.kv[l].K[:m]), (name, l)
            assert np.array_equal(o.target.kv[l].V[:m], ar.kv[l].V[:m]), (name, l)
        # closed-form cycle count
        R = _rejects_before_last(logs, w.G)
        assert len(logs) == schedule.cycle_count(w.n, w.G, R), name


@pytest.mark.parametrize("mi", [0, 2, 3])
def test_kv_lengths_and_rollback(mi):
    w, W, prompt, u = _setup(G=16, **MODELS[mi])
    ref, _ = ar_greedy(w, W, prompt, w.G)
    o = SPDOracle(w, W, policy=ForcedPolicy(ref, 0.6, u, w.V), uniforms=u)
    _, logs = o.run(prompt, w.G)
    per = w.L // w.n
    saw_reject = saw_full = False
    for l in logs:
        t, a = l["t"], l["a"]
        if l["exit_pos"] >= 0 and not l["accept"]:
            saw_reject = True
            assert l["kv_len"] == [l["exit_pos"] + 1] * w.L
        else:
            saw_full |= a == w.n
            exp = [t + 1 - min(layer // per, a) for layer in range(w.L)]
            assert l["kv_len"] == exp, l
        assert 1 <= a <= w.n
        assert l["depths"] == schedule.depth_layout(a, bool(l["pending_row"]), w.n)
    assert saw_reject and saw_full


def test_pdm_committed_length_tracks_verified_prefix():
    w, W, prompt, u = _setup(G=16, **MODELS[0])
    ref, _ = ar_greedy(w, W, prompt, w.G)
    o = SPDOracle(w, W, policy=ForcedPolicy(ref, 0.5, u, w.V), uniforms=u)
    _, logs = o.run(prompt, w.G)
    prev_exit = None
    for l in logs:
        # committed features = verified positions up to the previous exit
        if prev_exit is not None:
            assert l["pdm_len"] == prev_exit + 1
        else:
            assert l["pdm_len"] >= w.P
        if l["exit_pos"] >= 0:
            prev_exit = l["exit_pos"]
            # the next row to commit is this exit, at the committed length
            assert l["exit_pos"] == l["pdm_len"]


@pytest.mark.parametrize("mi", [0, 3, 4])
def test_incremental_pdm_equals_full_recompute(mi):
    w, W, prompt, u = _setup(G=12, **MODELS[mi])
    ref, _ = ar_greedy(w, W, prompt, w.G)
    o = SPDOracle(w, W, policy=ForcedPolicy(ref, 0.5, u, w.V), uniforms=u)
    checked = []

    def hook(kind, info):
        if kind != "pdm":
            return
        rows = info["rows"]
        C = rows[0][0]
        # full-depth anchors of the committed prefix from a fresh AR pass
        tgt = Target(w, W)
        feats = []
        pdm = PDM(w, W)
        for p in range(C):
            _, taps = tgt.forward_token(o.tokens[p], p)
            feats.append(pdm.feature(taps, w.n))
        full = np.concatenate([np.stack(feats), info["G"]]) if feats else info["G"]
        X = pdm.run_rows(full, 0)
        np.testing.assert_allclose(pdm.logits(X[-1]), info["logits"], rtol=1e-5, atol=1e-6)
        checked.append(info["cycle"])

    o.hook = hook
    o.run(prompt, w.G)
    assert len(checked) == len(o.logs)


def test_tiny_fp32_natural_run_is_autoregressive_pace():
    w = si.workload("tiny_fp32", G=20)
    W = si.nest_weights(si.weights_numpy_f32(si.make_weights(w)), w)
    prompt = si.make_prompt(w)
    o = SPDOracle(w, W)
    toks, logs = o.run(prompt, w.G)
    ref, _ = ar_greedy(w, W, prompt, w.G)
    assert toks == ref
    R = _rejects_before_last(logs, w.G)
    assert len(logs) == schedule.cycle_count(w.n, w.G, R)


def test_all_accepted_run_emits_one_token_per_cycle():
    w, W, prompt, u = _setup(G=20, **MODELS[2])
    ref, _ = ar_greedy(w, W, prompt, w.G)
    _, logs = SPDOracle(w, W, policy=ForcedPolicy(ref, 1.0, u, w.V), uniforms=u).run(prompt, w.G)
    assert len(logs) == w.n + w.G - 2
    K = len(logs)
    alpha = (w.G - 1) / K
    # equivalent acceptance length alpha * n approaches n as G grows
    assert alpha * w.n == pytest.approx(w.n * (w.G - 1) / (w.n + w.G - 2))


# -- planted mistakes: the pins above must catch them --------------------------

def _run_mutated(monkeypatch, attr, fn, mi=0):
    w, W, prompt, u = _setup(G=14, **MODELS[mi])
    ref, _ = ar_greedy(w, W, prompt, w.G)
    monkeypatch.setattr(*attr, fn)
    try:
        toks, _ = SPDOracle(w, W, policy=ForcedPolicy(ref, 0.5, u, w.V), uniforms=u).run(prompt, w.G)
    except AssertionError:
        return "assert"
    except (ValueError, TypeError):
        return "error"
    return "same" if toks == ref else "differs"


@pytest.mark.parametrize("delta", [-1, +1])
def test_wrong_truncation_length_is_caught(monkeypatch, delta):
    orig = Target.truncate

    def bad(self, length):
        return orig(self, length + delta)
    assert _run_mutated(monkeypatch, (Target, "truncate"), bad) != "same"


def test_dropped_feature_commit_is_caught(monkeypatch):
    orig = PDM.commit

    def bad(self, count):
        return orig(self, 0 if count == 1 else count)
    assert _run_mutated(monkeypatch, (PDM, "commit"), bad) == "assert"


def test_stage_skipping_a_layer_is_caught(monkeypatch):
    # a stage that runs one layer too few: AR is untouched, SPD must notice
    from oracle import model

    def bad(k, L, n, split=None):
        per = L // n
        return range(k * per, (k + 1) * per - 1)
    assert _run_mutated(monkeypatch, (model, "stage_layers"), bad, mi=2) != "same"
