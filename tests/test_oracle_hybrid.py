"""Pins of the oracle's hybrid target (linear-attention layers).

The pages ([RB] limitations, [TW] §11) say only that the 4B/9B targets
interleave one standard and three faster linear-attention layers per block of
four.  Reading taken: layer l is standard attention iff l % P == P - 1; the
others use textbook kernelised causal linear attention with feature map
phi = elu + 1, same projections, RoPE and KV cache.  What pins it:
  * linear_attention equals the recurrent form a decoder would run (a state
    S = sum_i phi(k_i) v_i^T and z = sum_i phi(k_i) updated one position at a
    time, output phi(q)^T S / phi(q)^T z) and a pure-Python triple loop;
  * the matrix and row forms of a hybrid layer agree;
  * the SPD state machine over hybrid targets stays lossless for every draft
    policy (tokens and KV equal greedy autoregressive decoding) with the same
    closed-form cycle count;
  * the layer-type rule puts one standard layer in every block of P.
"""
import numpy as np
import pytest

import seeded_inputs as si
from oracle import SPDOracle, ar_greedy, schedule
from oracle import model as M
from oracle.layers import elu_plus_one, linear_attention
from tests.test_oracle_spd import _policies

rng = np.random.default_rng(91)


def test_elu_plus_one_is_positive_and_continuous():
    x = np.array([-30.0, -1.0, -1e-7, 0.0, 1e-7, 2.5], np.float32)
    y = elu_plus_one(x)
    assert (y > 0).all()
    np.testing.assert_allclose(y, [np.exp(-30.0), np.exp(-1.0), np.exp(-1e-7), 1.0, 1.0 + 1e-7, 3.5], rtol=1e-6)


@pytest.mark.parametrize("Hq,Hkv,hd,T", [(2, 1, 4, 1), (4, 2, 8, 7), (6, 3, 16, 33)])
def test_linear_attention_equals_recurrent_state_form(Hq, Hkv, hd, T):
    q = rng.standard_normal((Hq, hd)).astype(np.float32)
    K = rng.standard_normal((T, Hkv, hd)).astype(np.float32)
    V = rng.standard_normal((T, Hkv, hd)).astype(np.float32)
    got = linear_attention(q, K, V)
    G = Hq // Hkv
    for h in range(Hq):
        kv = h // G
        S = np.zeros((hd, hd))
        z = np.zeros(hd)
        for i in range(T):  # one position at a time, float64
            fk = elu_plus_one(K[i, kv]).astype(np.float64)
            S += np.outer(fk, V[i, kv].astype(np.float64))
            z += fk
        fq = elu_plus_one(q[h]).astype(np.float64)
        np.testing.assert_allclose(got[h], (fq @ S) / (fq @ z), rtol=2e-5, atol=1e-6)


def test_linear_attention_brute_force_loops():
    Hq, Hkv, hd, T = 2, 1, 3, 4
    q = rng.standard_normal((Hq, hd)).astype(np.float32)
    K = rng.standard_normal((T, Hkv, hd)).astype(np.float32)
    V = rng.standard_normal((T, Hkv, hd)).astype(np.float32)
    phi = lambda x: x + 1.0 if x > 0 else float(np.exp(x))
    got = linear_attention(q, K, V)
    for h in range(Hq):
        w = [sum(phi(float(q[h, c])) * phi(float(K[i, 0, c])) for c in range(hd)) for i in range(T)]
        for j in range(hd):
            want = sum(w[i] * float(V[i, 0, j]) for i in range(T)) / sum(w)
            assert abs(got[h, j] - want) < 1e-5 * (1 + abs(want))


@pytest.mark.parametrize("P,L,want", [(4, 8, [0, 0, 0, 1, 0, 0, 0, 1]), (2, 4, [0, 1, 0, 1]), (0, 3, [1, 1, 1]),
                                      (1, 3, [1, 1, 1])])
def test_layer_type_rule(P, L, want):
    w = si.tiny(L=L, n=1, Ls=1, anchors=[0, L], attn_period=P)
    s = M._Shape(w)
    assert [int(not s.linear(l)) for l in range(L)] == want


def test_hybrid_layer_matrix_equals_rows():
    w = si.tiny(Hq=4, Hkv=2, L=2, n=1, Ls=1, anchors=[0, 1], attn_period=2)
    W = si.nest_weights(si.weights_numpy_f32(si.make_weights(w)), w)
    s = M._Shape(w)
    X = rng.standard_normal((6, w.d)).astype(np.float32)
    pre = rng.standard_normal((3, w.d)).astype(np.float32)
    kv1 = M.KVCache(w.max_ctx, w.Hkv, w.hd, False)
    kv2 = M.KVCache(w.max_ctx, w.Hkv, w.hd, False)
    M.layer_rows(s, W["layers"][0], pre, 0, kv1, linear=True)
    M.layer_rows(s, W["layers"][0], pre, 0, kv2, linear=True)
    a = M.layer_rows(s, W["layers"][0], X, 3, kv1, linear=True)
    b = M.layer_matrix(s, W["layers"][0], X, 3, kv2, linear=True)
    np.testing.assert_allclose(a, b, rtol=2e-5, atol=2e-6)
    # and it differs from the softmax layer on the same input
    kv3 = M.KVCache(w.max_ctx, w.Hkv, w.hd, False)
    M.layer_rows(s, W["layers"][0], pre, 0, kv3)
    c = M.layer_rows(s, W["layers"][0], X, 3, kv3)
    assert np.abs(a - c).max() > 1e-4


HYBRID = [
    dict(L=4, n=2, Ls=1, anchors=[0, 2, 3], Hq=4, Hkv=2, seed=61, attn_period=2),
    dict(L=8, n=4, Ls=2, anchors=[0, 2, 4, 6, 7], Hq=4, Hkv=4, seed=62, dtype="bf16", attn_period=4),
    dict(L=8, n=2, Ls=1, anchors=[0, 3, 8], Hq=6, Hkv=3, seed=63, norm_gain="random", attn_period=4),
    dict(L=4, n=1, Ls=2, anchors=[0, 2, 4], Hq=2, Hkv=1, seed=64, attn_period=4),
]


@pytest.mark.parametrize("mi", range(len(HYBRID)))
def test_hybrid_spd_is_lossless(mi):
    w = si.tiny(G=14, **HYBRID[mi])
    W = si.nest_weights(si.weights_numpy_f32(si.make_weights(w)), w)
    prompt, u = si.make_prompt(w), si.make_uniforms(w)
    ref, ar = ar_greedy(w, W, prompt, w.G)
    for name, pol in _policies(w, ref, u).items():
        o = SPDOracle(w, W, policy=pol, uniforms=u)
        toks, logs = o.run(prompt, w.G)
        assert toks == ref, name
        upto = len(ref) - 1
        for l in range(w.L):
            m = min(upto, o.target.kv[l].length)
            assert np.array_equal(o.target.kv[l].K[:m], ar.kv[l].K[:m]), (name, l)
        ver = [x for x in logs if x["exit_pos"] >= 0]
        R = sum(1 for x in ver[: w.G - 2] if not x["accept"])
        assert len(logs) == schedule.cycle_count(w.n, w.G, R), name


def test_hybrid_target_differs_from_the_all_softmax_target():
    kw = dict(HYBRID[0])
    w = si.tiny(G=10, **kw)
    W = si.nest_weights(si.weights_numpy_f32(si.make_weights(w)), w)
    prompt = si.make_prompt(w)
    h1, _ = M.Target(w, W).prefill_matrix(prompt)
    h2, _ = M.Target(w.replace(attn_period=0), W).prefill_matrix(prompt)
    assert np.abs(h1 - h2).max() > 1e-4
