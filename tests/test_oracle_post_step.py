"""Pins of the oracle's post-step schedule (the scheduling ablation of [PL] §4).

Under the post-step schedule the draft module reads the features after the
stage step.  What must hold, independently of how the oracle is written:
  * losslessness: for every draft policy the emitted tokens equal plain
    greedy autoregressive decoding, and the cycle count follows the same
    closed form as the pre-step schedule (the token flow is unchanged);
  * the rows are the pre-step rows one stage deeper: for a policy that does
    not look at the draft module, post-step cycle c sees exactly the rows
    (positions, depths and features) that pre-step cycle c+1 sees minus its
    newest one, and the draft module's hidden state of post-step cycle c's
    newest row equals that of the same row in pre-step cycle c+1 (the
    pre-step rows are pinned by [PL] §A.3's key-depth rule elsewhere);
  * every exit is committed in its own cycle: no row waits for the next one.
"""
import numpy as np
import pytest

import seeded_inputs as si
from oracle import SPDOracle, ForcedPolicy, NaturalPolicy, ar_greedy, schedule
from oracle.model import PDM, Target
from oracle.spd import FixedPolicy

MODELS = [
    dict(L=4, n=2, Ls=1, anchors=[0, 2, 3], Hq=4, Hkv=2, seed=21),
    dict(L=6, n=3, Ls=2, anchors=[0, 1, 4, 6], Hq=4, Hkv=1, seed=22),
    dict(L=8, n=4, Ls=2, anchors=[0, 2, 4, 6, 7], Hq=4, Hkv=4, seed=23, dtype="bf16"),
    dict(L=8, n=8, Ls=1, anchors=[0, 3, 8], Hq=6, Hkv=3, seed=24, norm_gain="random"),
]


def _setup(**kw):
    w = si.tiny(**kw)
    W = si.nest_weights(si.weights_numpy_f32(si.make_weights(w)), w)
    return w, W, si.make_prompt(w), si.make_uniforms(w)


def _policies(w, ref, u):
    G = len(ref)
    rng = np.random.default_rng(w.seed + 100)
    return {
        "natural": NaturalPolicy(),
        "right": ForcedPolicy(ref, 1.0, u, w.V),
        "wrong": ForcedPolicy(ref, 0.0, u, w.V),
        "p0.5": ForcedPolicy(ref, 0.5, u, w.V),
        "random": FixedPolicy(ref, list(rng.random(G) < 0.6), w.V),
    }


@pytest.mark.parametrize("mi", range(len(MODELS)))
def test_post_step_is_lossless(mi):
    w, W, prompt, u = _setup(G=14, **MODELS[mi])
    wp = w.replace(schedule="post")
    ref, ar = ar_greedy(w, W, prompt, w.G)
    for name, pol in _policies(w, ref, u).items():
        o = SPDOracle(wp, W, policy=pol, uniforms=u)
        toks, logs = o.run(prompt, w.G)
        assert toks == ref, name
        upto = len(ref) - 1
        for l in range(w.L):
            m = min(upto, o.target.kv[l].length)
            assert np.array_equal(o.target.kv[l].K[:m], ar.kv[l].K[:m]), (name, l)
        ver = [x for x in logs if x["exit_pos"] >= 0]
        R = sum(1 for x in ver[: w.G - 2] if not x["accept"])
        assert len(logs) == schedule.cycle_count(w.n, w.G, R), name


@pytest.mark.parametrize("mi", [0, 2])
def test_post_step_depths_and_commits(mi):
    w, W, prompt, u = _setup(G=16, **MODELS[mi])
    ref, _ = ar_greedy(w, W, prompt, w.G)
    o = SPDOracle(w.replace(schedule="post"), W, policy=ForcedPolicy(ref, 0.6, u, w.V), uniforms=u)
    _, logs = o.run(prompt, w.G)
    saw_exit = saw_reject = False
    for x in logs:
        a, t = x["a"], x["t"]
        # one stage deeper than at entry; the newest token has done stage 1
        assert x["depths"] == list(range(a, 0, -1))
        assert x["pending_row"] == 0
        if x["exit_pos"] >= 0:
            saw_exit = True
            saw_reject |= not x["accept"]
            assert a == w.n and x["exit_pos"] == t - w.n + 1
            # committed through the exited position in the same cycle
            assert x["pdm_len"] == x["exit_pos"] + 1
        else:
            assert x["pdm_len"] == t - a + 1
    assert saw_exit and saw_reject


class BlindPolicy:
    """Drafts that never look at the draft module: ref[q] where right[q], else
    ref[q] + 1 (mod V); 0 beyond the reference."""

    def __init__(self, ref, right, V):
        self.ref, self.right, self.V = list(ref), list(right), V

    def draft(self, q: int, pdm_tok: int) -> int:
        if q >= len(self.ref):
            return 0
        return self.ref[q] if self.right[q] else (self.ref[q] + 1) % self.V


@pytest.mark.parametrize("mi", [0, 1, 2, 3])
@pytest.mark.parametrize("pname", ["right", "random"])
def test_post_rows_are_next_pre_rows_minus_newest(mi, pname):
    """Policies that ignore the draft module give both schedules the same token
    flow; the post-step rows of cycle c must then be the pre-step rows of
    cycle c+1 without the entering token, features and hidden states alike."""
    w, W, prompt, u = _setup(G=14, **MODELS[mi])
    ref, _ = ar_greedy(w, W, prompt, w.G)
    seen = {"pre": {}, "post": {}}
    G = len(ref)
    right = [True] * G if pname == "right" else list(np.random.default_rng(w.seed + 7).random(G) < 0.6)

    def run(sched):
        pol = BlindPolicy(ref, right, w.V)
        o = SPDOracle(w.replace(schedule=sched), W, policy=pol, uniforms=u)

        def hook(kind, info):
            if kind == "pdm":
                seen[sched][info["cycle"]] = info
        o.hook = hook
        return o.run(prompt, w.G)

    tpre, lpre = run("pre")
    tpost, lpost = run("post")
    assert tpre == tpost == ref
    assert [x["a"] for x in lpre] == [x["a"] for x in lpost]
    assert [x["exit_pos"] for x in lpre] == [x["exit_pos"] for x in lpost]
    checked = 0
    for x in lpost[:-1]:
        c = x["cycle"]
        if x["exit_pos"] >= 0 and not x["accept"]:
            continue  # the flushed rows do not reappear
        po, pr = seen["post"][c], seen["pre"][c + 1]
        assert pr["rows"][:-1] == po["rows"], (c, pr["rows"], po["rows"])
        assert pr["rows"][-1][1] == 0
        np.testing.assert_allclose(po["G"], pr["G"][:-1], rtol=1e-6, atol=1e-7)
        np.testing.assert_allclose(po["X"][-1], pr["X"][-2], rtol=1e-4, atol=1e-5)
        checked += 1
    assert checked >= len(lpost) // 2


@pytest.mark.parametrize("mi", [0, 3])
def test_post_incremental_pdm_equals_full_recompute(mi):
    w, W, prompt, u = _setup(G=12, **MODELS[mi])
    ref, _ = ar_greedy(w, W, prompt, w.G)
    o = SPDOracle(w.replace(schedule="post"), W, policy=ForcedPolicy(ref, 0.5, u, w.V), uniforms=u)
    checked = []

    def hook(kind, info):
        if kind != "pdm":
            return
        C = info["rows"][0][0]
        tgt = Target(w, W)
        pdm = PDM(w, W)
        feats = []
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


def test_post_step_needs_two_stages():
    w, W, prompt, u = _setup(G=6, L=4, n=1, Ls=1, anchors=[0, 2, 4], seed=25)
    with pytest.raises(ValueError):
        SPDOracle(w.replace(schedule="post"), W, uniforms=u)
