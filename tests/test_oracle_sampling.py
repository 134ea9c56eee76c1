"""Pins of the oracle's temperature-1 rejection-sampling verification (CPU only)."""
import numpy as np
import pytest

import seeded_inputs as si
from oracle import SPDOracle, sampling
from oracle.model import Target

rng = np.random.default_rng(5)


def _rand_dist(V, zeros=0):
    p = rng.random(V) ** 3
    if zeros:
        p[rng.choice(V, zeros, replace=False)] = 0
    return p / p.sum()


@pytest.mark.parametrize("V,zq,zp", [(2, 0, 0), (5, 0, 0), (8, 2, 0), (8, 0, 3), (7, 1, 1)])
def test_rejection_rule_emits_target_distribution_exactly(V, zq, zp):
    for _ in range(20):
        P, Q = _rand_dist(V, zp), _rand_dist(V, zq)
        np.testing.assert_allclose(sampling.emit_distribution(P, Q), P, rtol=0, atol=1e-12)


def test_identical_draft_distribution_is_always_accepted():
    P = _rand_dist(6)
    np.testing.assert_allclose(sampling.emit_distribution(P, P), P, atol=1e-15)
    w = P.astype(np.float32)
    for x in range(6):
        for u in (0.0, 0.5, 1 - 2 ** -24):
            assert sampling.accept_test(w, float(w.astype(np.float64).sum()), w,
                                        float(w.astype(np.float64).sum()), x, u)[0]


def test_inverse_cdf_boundaries():
    w = np.array([0, 1, 0, 3], np.float32)
    assert sampling.inverse_cdf(w, 0.0)[0] == 1
    assert sampling.inverse_cdf(w, 0.2499)[0] == 1
    assert sampling.inverse_cdf(w, 0.25)[0] == 3  # cumsum must strictly exceed u * total
    assert sampling.inverse_cdf(w, 1 - 2 ** -24)[0] == 3


def test_oracle_sampling_functions_integrate_to_target():
    """Drive the oracle's own inverse-CDF, acceptance test and residual with
    uniform grids; the emitted law must equal P to grid accuracy."""
    V, N = 7, 4096
    grid = (np.arange(N) + 0.5) / N
    for _ in range(5):
        lp = rng.standard_normal(V).astype(np.float32) * 2
        lq = rng.standard_normal(V).astype(np.float32) * 2
        pw, pZ = sampling.softmax_weights(lp)
        qw, qZ = sampling.softmax_weights(lq)
        Qx = np.bincount([sampling.inverse_cdf(qw, u)[0] for u in grid], minlength=V) / N
        r = sampling.residual(pw, pZ, qw, qZ)
        rlaw = np.bincount([sampling.inverse_cdf(r, u)[0] for u in grid], minlength=V) / N
        emit = np.zeros(V)
        for x in range(V):
            acc = np.mean([sampling.accept_test(pw, pZ, qw, qZ, x, u)[0] for u in grid])
            emit[x] += Qx[x] * acc
            emit += Qx[x] * (1 - acc) * rlaw
        P = pw.astype(np.float64) / pZ
        np.testing.assert_allclose(emit, P, atol=4.0 / N)


def test_softmax_weights_match_definition():
    l = rng.standard_normal(50).astype(np.float32) * 3
    w, Z = sampling.softmax_weights(l)
    ref = np.exp(l.astype(np.float64) - l.max())
    np.testing.assert_allclose(w, ref, rtol=1e-6)
    assert Z == pytest.approx(ref.sum(), rel=1e-6)


def _first_two_tokens_chi2(top_k: int = 0):
    w = si.tiny(L=2, n=2, Ls=1, anchors=[0, 2], d=32, Hq=2, Hkv=1, hd=16, F=48, V=11,
                P=4, G=2, mode="sample", seed=21, top_k=top_k)
    W = si.nest_weights(si.weights_numpy_f32(si.make_weights(w)), w)
    W["lm_head"] = W["lm_head"] * np.float32(25.0)       # sharpen P
    W["pdm_lm_head"] = W["pdm_lm_head"] * np.float32(25.0)  # a different, sharp Q
    prompt = si.make_prompt(w)
    # exact autoregressive joint law p(x_P) p(x_P+1 | x_P)
    tgt = Target(w, W)
    for p, tok in enumerate(prompt):
        h, _ = tgt.forward_token(int(tok), p)
    lp1 = tgt.logits(h)
    w1, Z1 = sampling.softmax_weights(lp1, 1.0, top_k)
    P1 = w1.astype(np.float64) / Z1
    joint = np.zeros((w.V, w.V))
    for x in range(w.V):
        t2 = Target(w, W)
        for p, tok in enumerate(list(prompt) + [x]):
            h2, _ = t2.forward_token(int(tok), p)
        w2, Z2 = sampling.softmax_weights(t2.logits(h2), 1.0, top_k)
        joint[x] = P1[x] * w2.astype(np.float64) / Z2
    runs = 4000
    counts = np.zeros((w.V, w.V))
    rejects = 0
    for s in range(runs):
        u = si.make_uniforms(w, seed=1000 + s)
        o = SPDOracle(w, W, uniforms=u)
        toks, logs = o.run(prompt, 2)
        counts[toks[w.P], toks[w.P + 1]] += 1
        rejects += sum(1 for l in logs if l["exit_pos"] >= 0 and not l["accept"])
    assert 0.05 * runs < rejects < 0.95 * runs  # both branches exercised
    exp = joint * runs
    mask = exp >= 5
    chi2 = float((((counts - exp) ** 2)[mask] / exp[mask]).sum())
    dof = int(mask.sum()) - 1
    # 1e-4 upper tail of chi-square via Wilson-Hilferty
    z = 3.719
    crit = dof * (1 - 2 / (9 * dof) + z * np.sqrt(2 / (9 * dof))) ** 3
    return chi2, crit, counts[~mask].sum(), exp[~mask].sum()


@pytest.mark.slow
@pytest.mark.parametrize("top_k", [0, 3])
def test_spd_sampling_first_tokens_follow_autoregressive_law(top_k):
    """Chi-square test: the joint law of the first two generated tokens under
    SPD with rejection sampling equals the target's autoregressive law (with
    top-k: the autoregressive law of the truncated target)."""
    chi2, crit, tail_n, tail_e = _first_two_tokens_chi2(top_k)
    assert chi2 < crit, (chi2, crit)
    assert tail_n <= tail_e * 3 + 10


@pytest.mark.slow
def test_resampling_from_target_instead_of_residual_is_caught(monkeypatch):
    """Planted mistake: redrawing a rejected token from P (not max(0, P-Q))
    biases the output; the chi-square test above must see it."""
    monkeypatch.setattr(sampling, "residual",
                        lambda pw, pZ, qw, qZ: pw.astype(np.float64) / pZ)
    chi2, crit, _, _ = _first_two_tokens_chi2()
    assert chi2 > crit


@pytest.mark.parametrize("T", [1.0, 0.5])
def test_shift_bounds_hold_under_logit_perturbations(T):
    """cdf_shift_bound, accept_shift_bound and residual_shift_bound bound the
    movement of every inverse-CDF boundary, of the accept-test gap and of the
    residual's CDF when each logit moves by at most eps (random and
    worst-case-signed perturbations)."""
    for trial in range(200):
        V = int(rng.integers(2, 60))
        eps = float(rng.choice([1e-4, 1e-3, 1e-2, 5e-2]))
        lp = rng.standard_normal(V).astype(np.float32) * 2
        lq = rng.standard_normal(V).astype(np.float32) * 2
        if trial % 2:
            dp = rng.uniform(-eps, eps, V)
            dq = rng.uniform(-eps, eps, V)
        else:  # all mass below one boundary up, all above it down
            cut = int(rng.integers(0, V))
            dp = np.where(np.arange(V) <= cut, eps, -eps)
            dq = -dp
        pw, pZ = sampling.softmax_weights(lp, T)
        qw, qZ = sampling.softmax_weights(lq, T)
        pw2, pZ2 = sampling.softmax_weights((lp + dp).astype(np.float32), T)
        qw2, qZ2 = sampling.softmax_weights((lq + dq).astype(np.float32), T)
        # every boundary of the inverse CDF
        c1 = np.cumsum(qw.astype(np.float64)) / qZ
        c2 = np.cumsum(qw2.astype(np.float64)) / qZ2
        assert np.max(np.abs(c1 - c2)) <= sampling.cdf_shift_bound(eps * 1.0001, T) + 1e-7
        # the accept test's gap
        P, Q = pw.astype(np.float64) / pZ, qw.astype(np.float64) / qZ
        P2, Q2 = pw2.astype(np.float64) / pZ2, qw2.astype(np.float64) / qZ2
        x = int(rng.integers(0, V))
        u = float(rng.random())
        moved = abs((u * Q2[x] - P2[x]) - (u * Q[x] - P[x])) / Q[x]
        assert moved <= sampling.accept_shift_bound(eps * 1.0001, eps * 1.0001, P[x], Q[x], u, T) + 1e-7
        # the residual's CDF
        r1, r2 = np.maximum(0, P - Q), np.maximum(0, P2 - Q2)
        if r1.sum() > 0 and r2.sum() > 0:
            b = sampling.residual_shift_bound(eps * 1.0001, eps * 1.0001, P, Q, T)
            d = np.max(np.abs(np.cumsum(r1) / r1.sum() - np.cumsum(r2) / r2.sum()))
            assert d <= b + 1e-7
