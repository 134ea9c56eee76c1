"""Pins of the oracle's heads, anchor fusion and temperature softmax (CPU only).

These functions are shared by the oracle's SPD run and its autoregressive
reference, so the lossless tests cannot see a mistake in them.  Each is pinned
here against something other than itself:

  * the target's final RMSNorm + LM head: a torch composition of the whole
    tiny model (embedding, every layer, rms_norm with random gains, matmul);
  * the draft module's head: torch rms_norm + matmul with random gains
    ([PL] §3.1: the module has its own LM head);
  * the anchor-fusion feature g(p, k) ([RB] core method: the reachable
    anchors are concatenated and projected by the FC of the depth's pattern):
    torch.cat + matmul, the block-sum form over anchors, the depth-0 case
    ([PL] §3.2: depth 0 reduces to a projection of the embedding), and the
    property that anchors beyond f(k) do not enter;
  * the temperature softmax: torch.softmax(l / T), and a chi-square test of
    the first SPD tokens against the autoregressive law at T = 0.5 whose
    expected law is built with torch's softmax.

Every pin comes with a planted mistake (monkeypatched into the oracle) that
the same check must catch.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as Fn

import seeded_inputs as si
from oracle import SPDOracle, sampling
from oracle import model as M
from oracle.layers import rmsnorm
from oracle.schedule import pattern

from test_oracle_layers import _torch_layer

rng = np.random.default_rng(31)


def _model(**kw):
    w = si.tiny(**kw)
    return w, si.nest_weights(si.weights_numpy_f32(si.make_weights(w)), w)


# ---------------------------------------------------------------------------
# target: final norm + LM head
# ---------------------------------------------------------------------------
def _torch_logits(w, W, toks):
    """Logits of every position: embedding -> L torch layers -> rms_norm -> LM head."""
    X = W["embed"][np.asarray(toks)].astype(np.float32)
    for l in range(w.L):
        X = _torch_layer(w, W["layers"][l], X)
    T_ = torch.from_numpy
    U = Fn.rms_norm(T_(X), (w.d,), weight=T_(W["final_norm"]), eps=w.eps)
    return (U @ T_(W["lm_head"]).T).numpy()


def _target_logit_gap(w, W, toks):
    ref = _torch_logits(w, W, toks)
    tgt = M.Target(w, W)
    worst = 0.0
    for p, t in enumerate(toks):
        h, _ = tgt.forward_token(int(t), p)
        lg = tgt.logits(h)
        worst = max(worst, float(np.max(np.abs(lg - ref[p])) / np.max(np.abs(ref[p]))))
    return worst


@pytest.mark.parametrize("Hq,Hkv", [(4, 2), (4, 4)])
def test_target_logits_match_torch_whole_model(Hq, Hkv):
    w, W = _model(Hq=Hq, Hkv=Hkv, norm_gain="random", L=3, n=1, Ls=1, anchors=[0, 1], P=7, seed=41)
    toks = [int(t) for t in si.make_prompt(w)]
    assert _target_logit_gap(w, W, toks) < 2e-4


def test_dropped_final_norm_is_caught(monkeypatch):
    w, W = _model(norm_gain="random", L=3, n=1, Ls=1, anchors=[0, 1], P=7, seed=41)
    toks = [int(t) for t in si.make_prompt(w)]
    monkeypatch.setattr(M.Target, "logits", lambda self, h: self.W["lm_head"] @ h)
    assert _target_logit_gap(w, W, toks) > 1e-2


def test_target_logits_rows_match_torch():
    w, W = _model(norm_gain="random", seed=42)
    H = rng.standard_normal((6, w.d)).astype(np.float32)
    T_ = torch.from_numpy
    ref = (Fn.rms_norm(T_(H), (w.d,), weight=T_(W["final_norm"]), eps=w.eps) @ T_(W["lm_head"]).T).numpy()
    np.testing.assert_allclose(M.Target(w, W).logits_rows(H), ref, rtol=1e-4, atol=1e-5)


# ---------------------------------------------------------------------------
# draft module: head
# ---------------------------------------------------------------------------
def _pdm_head_gap(w, W):
    pdm = M.PDM(w, W)
    T_ = torch.from_numpy
    worst = 0.0
    for _ in range(5):
        x = rng.standard_normal(w.d).astype(np.float32) * 3
        ref = (Fn.rms_norm(T_(x), (w.d,), weight=T_(W["pdm_final_norm"]), eps=w.eps)
               @ T_(W["pdm_lm_head"]).T).numpy()
        worst = max(worst, float(np.max(np.abs(pdm.logits(x) - ref)) / np.max(np.abs(ref))))
    return worst


def test_pdm_logits_match_torch():
    w, W = _model(norm_gain="random", seed=43)
    assert _pdm_head_gap(w, W) < 1e-5


@pytest.mark.parametrize("mistake", ["no_norm", "target_gain", "target_head"])
def test_pdm_head_mistakes_are_caught(monkeypatch, mistake):
    w, W = _model(norm_gain="random", seed=43)
    bad = {
        "no_norm": lambda self, x: self.W["pdm_lm_head"] @ x,
        "target_gain": lambda self, x: self.W["pdm_lm_head"] @ rmsnorm(x, self.W["final_norm"], self.s.eps),
        "target_head": lambda self, x: self.W["lm_head"] @ rmsnorm(x, self.W["pdm_final_norm"], self.s.eps),
    }[mistake]
    monkeypatch.setattr(M.PDM, "logits", bad)
    assert _pdm_head_gap(w, W) > 1e-3


# ---------------------------------------------------------------------------
# draft module: anchor fusion g(p, k) = W_fc[f(k)] concat(A[0..f(k)])
# ---------------------------------------------------------------------------
def _fusion_case():
    w, W = _model(L=8, n=4, anchors=[0, 2, 5, 8], seed=44)
    # distinct anchors of distinct scales, so that any mix-up of their order shows
    taps = [rng.standard_normal(w.d).astype(np.float32) * (1 + i) for i in range(len(w.anchors))]
    return w, W, M.PDM(w, W), taps


def _fusion_gap(w, W, pdm, taps):
    """Largest relative difference of the oracle's feature and its two
    independent forms, over every depth k."""
    T_ = torch.from_numpy
    worst = 0.0
    for k in range(w.n + 1):
        f = pattern(k, w.anchors, w.L, w.n)
        got = pdm.feature(taps, k)
        cat = (T_(W["fc"][f]) @ torch.cat([T_(taps[i]) for i in range(f + 1)])).numpy()
        blocks = sum(W["fc"][f][:, i * w.d:(i + 1) * w.d].astype(np.float64) @ taps[i].astype(np.float64)
                     for i in range(f + 1))
        rows = pdm.feature_rows([taps], k)[0]
        for ref in (cat, blocks, rows):
            worst = max(worst, float(np.max(np.abs(got - ref)) / np.max(np.abs(ref))))
    return worst


def test_feature_matches_concat_and_block_sum():
    assert _fusion_gap(*_fusion_case()) < 1e-5


def test_depth_zero_feature_is_the_embedding_projection():
    """[PL] §3.2: at depth 0 the feature is the FC projection of the embedding alone."""
    w, W, pdm, taps = _fusion_case()
    assert pattern(0, w.anchors, w.L, w.n) == 0
    ref = (torch.from_numpy(W["fc"][0]) @ torch.from_numpy(taps[0])).numpy()
    np.testing.assert_allclose(pdm.feature(taps, 0), ref, rtol=1e-5, atol=1e-7)
    assert W["fc"][0].shape == (w.d, w.d)


def test_feature_reads_exactly_the_reachable_anchors():
    """Anchors beyond f(k) leave g(p, k) bit-identical; anchor f(k) changes it."""
    w, W, pdm, taps = _fusion_case()
    for k in range(w.n + 1):
        f = pattern(k, w.anchors, w.L, w.n)
        base = pdm.feature(taps, k)
        for i in range(f + 1, len(taps)):
            t2 = list(taps)
            t2[i] = t2[i] + np.float32(5.0)
            assert np.array_equal(pdm.feature(t2, k), base), (k, i)
        t3 = list(taps)
        t3[f] = t3[f] + np.float32(5.0)
        assert not np.allclose(pdm.feature(t3, k), base), k


@pytest.mark.parametrize("mistake", ["reversed", "shifted", "last_pattern"])
def test_fusion_mistakes_are_caught(monkeypatch, mistake):
    w, W, pdm, taps = _fusion_case()

    def bad(self, tp, k):
        f = pattern(k, self.s.anchors, self.s.L, self.s.n)
        if mistake == "reversed":
            x = np.concatenate([tp[i] for i in range(f, -1, -1)])
        elif mistake == "shifted":  # off by one: anchors 1..f+1 (or the last f+1)
            lo = min(1, len(tp) - 1 - f)
            x = np.concatenate([tp[i] for i in range(lo, lo + f + 1)])
        else:  # every depth uses the full-depth projection's leading columns
            x = np.concatenate([tp[i] for i in range(f + 1)])
            return self.W["fc"][-1][:, : x.size] @ x
        return self.W["fc"][f] @ x.astype(np.float32)

    monkeypatch.setattr(M.PDM, "feature", bad)
    assert _fusion_gap(w, W, pdm, taps) > 1e-2


# ---------------------------------------------------------------------------
# temperature softmax
# ---------------------------------------------------------------------------
def _softmax_gap(T):
    worst = 0.0
    for _ in range(5):
        l = rng.standard_normal(300).astype(np.float32) * 3
        w, Z = sampling.softmax_weights(l, T)
        ref = torch.softmax(torch.from_numpy(l).double() / T, dim=0).numpy()
        worst = max(worst, float(np.max(np.abs(w.astype(np.float64) / Z - ref))))
    return worst


@pytest.mark.parametrize("T", [1.0, 0.7, 0.5, 0.3, 2.0])
def test_softmax_weights_match_torch_at_temperature(T):
    assert _softmax_gap(T) < 1e-6


def test_missing_temperature_is_caught(monkeypatch):
    orig = sampling.softmax_weights
    monkeypatch.setattr(sampling, "softmax_weights", lambda l, T=1.0, k=0, keep=None: orig(l, 1.0, k, keep))
    assert _softmax_gap(0.5) > 1e-3


def _chi2_first_two_tokens(T, runs=3000):
    """Joint law of the first two SPD tokens at temperature T against the
    autoregressive law built with torch.softmax(logits / T)."""
    w = si.tiny(L=2, n=2, Ls=1, anchors=[0, 2], d=32, Hq=2, Hkv=1, hd=16, F=48, V=9,
                P=4, G=2, mode="sample", seed=23, temperature=T)
    W = si.nest_weights(si.weights_numpy_f32(si.make_weights(w)), w)
    W["lm_head"] = W["lm_head"] * np.float32(10.0)
    W["pdm_lm_head"] = W["pdm_lm_head"] * np.float32(10.0)
    prompt = [int(t) for t in si.make_prompt(w)]

    def law(toks):
        tgt = M.Target(w, W)
        for p, tok in enumerate(toks):
            h, _ = tgt.forward_token(int(tok), p)
        return torch.softmax(torch.from_numpy(tgt.logits(h)).double() / T, dim=0).numpy()

    P1 = law(prompt)
    joint = np.stack([P1[x] * law(prompt + [x]) for x in range(w.V)])
    counts = np.zeros((w.V, w.V))
    rejects = 0
    for s in range(runs):
        o = SPDOracle(w, W, uniforms=si.make_uniforms(w, seed=5000 + s))
        toks, logs = o.run(prompt, 2)
        counts[toks[w.P], toks[w.P + 1]] += 1
        rejects += sum(1 for l in logs if l["exit_pos"] >= 0 and not l["accept"])
    exp = joint * runs
    mask = exp >= 5
    chi2 = float((((counts - exp) ** 2)[mask] / exp[mask]).sum())
    dof = int(mask.sum()) - 1
    z = 3.719  # 1e-4 upper tail, Wilson-Hilferty
    crit = dof * (1 - 2 / (9 * dof) + z * np.sqrt(2 / (9 * dof))) ** 3
    return chi2, crit, rejects / runs


@pytest.mark.slow
def test_spd_sampling_at_half_temperature_follows_autoregressive_law():
    chi2, crit, rej = _chi2_first_two_tokens(0.5)
    assert 0.05 < rej < 0.95
    assert chi2 < crit, (chi2, crit)


@pytest.mark.slow
def test_sampling_without_temperature_is_caught_by_chi_square(monkeypatch):
    orig = sampling.softmax_weights
    monkeypatch.setattr(sampling, "softmax_weights", lambda l, T=1.0, k=0, keep=None: orig(l, 1.0, k, keep))
    chi2, crit, _ = _chi2_first_two_tokens(0.5)
    assert chi2 > crit
