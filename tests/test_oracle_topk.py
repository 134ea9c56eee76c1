"""Pins of the oracle's top-k truncation ([RB] reproducibility assessment:
top-k 50, top-p 1.0 at evaluation).

  * the kept ids are the k largest logits with ties to the lower id -- brute
    force over tie-heavy inputs;
  * the truncated weights are the full softmax weights on the kept ids and 0
    elsewhere, i.e. P_k = P restricted to the top k and renormalised (closed
    form), and k >= V reproduces the full softmax;
  * top-k 1 turns sampling into greedy decoding: sampled SPD with k = 1 must
    emit exactly the target's greedy autoregressive continuation, every
    verification accepting iff the draft is the target's argmax;
  * the rejection rule on truncated P and Q emits P_k exactly (enumeration);
    the chi-square test of the first two SPD tokens against the truncated
    autoregressive law sits with the other sampling pins.
"""
import numpy as np
import pytest

import seeded_inputs as si
from oracle import SPDOracle, ar_greedy, sampling
from tests.test_oracle_spd import MODELS, _setup

rng = np.random.default_rng(77)


@pytest.mark.parametrize("V,k", [(1, 1), (7, 3), (20, 5), (64, 50), (200, 50), (50, 64)])
def test_top_k_ids_brute_force(V, k):
    for trial in range(20):
        if trial % 2:
            l = rng.integers(-3, 4, V).astype(np.float32)  # many ties
        else:
            l = rng.standard_normal(V).astype(np.float32)
        want = sorted(sorted(range(V), key=lambda i: (-float(l[i]), i))[:k])
        assert list(sampling.top_k_ids(l, k)) == want


@pytest.mark.parametrize("k", [1, 2, 5, 19, 20, 25])
def test_truncated_weights_closed_form(k):
    V = 20
    for T in (1.0, 0.7):
        l = (rng.standard_normal(V) * 2).astype(np.float32)
        l[3] = l[11]  # a tie somewhere
        w, Z = sampling.softmax_weights(l, T, k)
        wf, Zf = sampling.softmax_weights(l, T)
        kept = set(sampling.top_k_ids(l, k)) if k < V else set(range(V))
        for v in range(V):
            assert w[v] == (wf[v] if v in kept else 0.0)
        P = wf.astype(np.float64) / Zf
        Pk = np.array([P[v] if v in kept else 0.0 for v in range(V)])
        np.testing.assert_allclose(w.astype(np.float64) / Z, Pk / Pk.sum(), rtol=1e-6, atol=1e-12)
        if k >= V:
            assert np.array_equal(w, wf) and Z == Zf


def test_rejection_rule_on_truncated_distributions_emits_truncated_target():
    V, k = 9, 4
    for _ in range(20):
        lp = rng.standard_normal(V).astype(np.float32) * 2
        lq = rng.standard_normal(V).astype(np.float32) * 2
        pw, pZ = sampling.softmax_weights(lp, 1.0, k)
        qw, qZ = sampling.softmax_weights(lq, 1.0, k)
        P, Q = pw.astype(np.float64) / pZ, qw.astype(np.float64) / qZ
        np.testing.assert_allclose(sampling.emit_distribution(P, Q), P, rtol=0, atol=1e-12)
        assert np.count_nonzero(P) == k


@pytest.mark.parametrize("mi", [0, 2, 3, 4])
def test_top_k_one_sampling_is_greedy_decoding(mi):
    w, W, prompt, _ = _setup(G=12, mode="sample", top_k=1, **MODELS[mi])
    u = si.make_uniforms(w)
    ref, _ = ar_greedy(w, W, prompt, w.G)
    o = SPDOracle(w, W, uniforms=u)
    pdm_argmax = {}
    o.hook = lambda kind, info: pdm_argmax.__setitem__(info["cycle"], int(np.argmax(info["logits"]))) \
        if kind == "pdm" else None
    toks, logs = o.run(prompt, w.G)
    assert toks == ref
    for x in logs:
        # Q is truncated too: the draw from a one-point Q is the draft module's argmax
        assert x["pdm_raw"] == pdm_argmax[x["cycle"]]
        if x["exit_pos"] >= 0:
            assert x["accept"] == int(x["draft"] == ref[x["exit_pos"] + 1])


def test_top_k_set_gap_brute_force():
    """The gap of a candidate kept set is the smallest uniform logit
    perturbation bound under which it becomes the top-k set: brute force over
    every k-subset of a small vocabulary."""
    import itertools
    V, k = 7, 3
    for _ in range(30):
        l = rng.standard_normal(V).astype(np.float32)
        for S in itertools.combinations(range(V), k):
            out = [v for v in range(V) if v not in S]
            want = max(0.0, max(float(l[v]) for v in out) - min(float(l[v]) for v in S))
            assert sampling.top_k_set_gap(l, list(S)) == pytest.approx(want, abs=0)
        assert sampling.top_k_set_gap(l, sampling.top_k_ids(l, k)) == 0.0


def test_top_k_one_set_gap_is_the_argmax_rule():
    l = rng.standard_normal(50).astype(np.float32)
    for x in range(50):
        assert sampling.top_k_set_gap(l, [x]) == float(l.max()) - float(l[x])


def test_kept_set_teacher_validation():
    """A teacher's kept set is adopted when it is a near-tie, and a set that
    leaves out a clearly larger logit is a mismatch."""
    from oracle.spd import Decisions
    l = np.array([5.0, 4.0, 3.0, 2.99, 1.0, 0.0], np.float32)
    d = Decisions({("qset", 0): [0, 1, 3], ("qset", 1): [0, 1, 4], ("qset", 2): [0, 1, 2]}, tol=0.05)
    assert list(d.kept_set(("qset", 0), l, 3)) == [0, 1, 3] and len(d.adopted) == 1
    d.kept_set(("qset", 1), l, 3)
    assert len(d.mismatch) == 1
    assert list(d.kept_set(("qset", 2), l, 3)) == [0, 1, 2] and len(d.adopted) == 1


def test_softmax_weights_on_a_given_set():
    l = rng.standard_normal(30).astype(np.float32)
    keep = [1, 7, 8, 20]
    w, Z = sampling.softmax_weights(l, 0.7, keep=keep)
    wf, _ = sampling.softmax_weights(l, 0.7)
    for v in range(30):
        assert w[v] == (wf[v] if v in keep else 0.0)
    assert Z == pytest.approx(float(wf[keep].astype(np.float64).sum()), rel=1e-12)
