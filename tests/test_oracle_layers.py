"""Pins of the oracle's layer primitives against independent torch CPU routines
and mathematical properties (CPU only)."""
import numpy as np
import pytest
import torch
import torch.nn.functional as Fn

import seeded_inputs as si
from oracle import layers as Lr
from oracle import model as M

rng = np.random.default_rng(0)


def test_bf16_round_matches_torch():
    x = rng.standard_normal(100000).astype(np.float32) * np.float32(3.0)
    # exact ties and boundaries: mantissa patterns with low half 0x8000
    ties = (np.arange(1000, dtype=np.uint32) << np.uint32(16)) | np.uint32(0x8000)
    ties = (ties + np.uint32(0x3F800000)).view(np.float32)
    for v in (x, ties, np.array([0.0, -0.0, 1e-30, -65504.0, 3.3e38], np.float32)):
        ref = torch.from_numpy(v.copy()).to(torch.bfloat16).to(torch.float32).numpy()
        assert np.array_equal(Lr.bf16_round(v).view(np.uint32), ref.view(np.uint32))


def test_rmsnorm_matches_torch():
    x = rng.standard_normal(2560).astype(np.float32)
    g = (1 + 0.1 * rng.standard_normal(2560)).astype(np.float32)
    ref = Fn.rms_norm(torch.from_numpy(x), (2560,), weight=torch.from_numpy(g), eps=1e-6).numpy()
    np.testing.assert_allclose(Lr.rmsnorm(x, g, 1e-6), ref, rtol=2e-6, atol=1e-7)


def test_silu_matches_torch():
    x = rng.standard_normal(1000).astype(np.float32) * 5
    np.testing.assert_allclose(Lr.silu(x), Fn.silu(torch.from_numpy(x)).numpy(), rtol=1e-6, atol=1e-7)


def test_rope_equals_complex_rotation():
    hd, pos = 128, 777
    x = rng.standard_normal((3, hd)).astype(np.float32)
    c, s = Lr.rope_cos_sin(pos, hd, 10000.0)
    got = Lr.apply_rope(x, c, s)
    # independent form: z_i = x_i + 1j x_{i+hd/2} multiplied by exp(1j pos theta_i)
    theta = 10000.0 ** (-np.arange(hd // 2) * 2.0 / hd)
    z = (x[:, : hd // 2] + 1j * x[:, hd // 2:]).astype(np.complex128) * np.exp(1j * pos * theta)
    ref = np.concatenate([z.real, z.imag], axis=1)
    np.testing.assert_allclose(got, ref, rtol=1e-5, atol=1e-5)


def test_rope_dot_depends_only_on_relative_position():
    hd = 64
    q = rng.standard_normal(hd).astype(np.float32)
    k = rng.standard_normal(hd).astype(np.float32)

    def dot(pq, pk):
        cq, sq = Lr.rope_cos_sin(pq, hd, 10000.0)
        ck, sk = Lr.rope_cos_sin(pk, hd, 10000.0)
        return float(Lr.apply_rope(q, cq, sq) @ Lr.apply_rope(k, ck, sk))

    assert dot(10, 3) == pytest.approx(dot(107, 100), rel=1e-4, abs=1e-4)
    assert dot(0, 0) == pytest.approx(float(q @ k), rel=1e-5)


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (20, 4), (8, 2)])
def test_attention_matches_torch_sdpa(Hq, Hkv):
    hd, T = 32, 37
    q = rng.standard_normal((Hq, hd)).astype(np.float32)
    K = rng.standard_normal((T, Hkv, hd)).astype(np.float32)
    V = rng.standard_normal((T, Hkv, hd)).astype(np.float32)
    grp = Hq // Hkv
    tq = torch.from_numpy(q)[:, None, :]                            # [Hq, 1, hd]
    tk = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(grp, 0)  # [Hq, T, hd]
    tv = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(grp, 0)
    ref = Fn.scaled_dot_product_attention(tq, tk.contiguous(), tv.contiguous())[:, 0, :].numpy()
    np.testing.assert_allclose(Lr.attention(q, K, V), ref, rtol=1e-5, atol=1e-6)


def test_attention_single_key_returns_value():
    q = rng.standard_normal((4, 16)).astype(np.float32)
    K = rng.standard_normal((1, 2, 16)).astype(np.float32)
    V = rng.standard_normal((1, 2, 16)).astype(np.float32)
    out = Lr.attention(q, K, V)
    np.testing.assert_allclose(out, V[0][[0, 0, 1, 1]], rtol=1e-6)


def _torch_layer(w, lw, xs):
    """Independent whole-layer reference over a sequence, composed of torch ops."""
    T_ = torch.from_numpy
    X = T_(xs)
    Tn = X.shape[0]
    d, Hq, Hkv, hd, F = w.d, w.Hq, w.Hkv, w.hd, w.F
    u = Fn.rms_norm(X, (d,), weight=T_(lw["attn_norm"]), eps=w.eps)
    qkv = u @ T_(lw["w_qkv"]).T
    q = qkv[:, : Hq * hd].reshape(Tn, Hq, hd)
    k = qkv[:, Hq * hd:(Hq + Hkv) * hd].reshape(Tn, Hkv, hd)
    v = qkv[:, (Hq + Hkv) * hd:].reshape(Tn, Hkv, hd)
    pos = torch.arange(Tn, dtype=torch.float64)[:, None]
    theta = w.rope_base ** (-torch.arange(hd // 2, dtype=torch.float64) * 2 / hd)
    rot = torch.polar(torch.ones(Tn, hd // 2, dtype=torch.float64), pos * theta)[:, None, :]

    def rope(x):
        z = torch.complex(x[..., : hd // 2].double(), x[..., hd // 2:].double()) * rot
        return torch.cat([z.real, z.imag], -1).float()
    q, k = rope(q), rope(k)
    grp = Hq // Hkv
    kk = k.permute(1, 0, 2).repeat_interleave(grp, 0).contiguous()
    vv = v.permute(1, 0, 2).repeat_interleave(grp, 0).contiguous()
    o = Fn.scaled_dot_product_attention(q.permute(1, 0, 2).contiguous(), kk, vv, is_causal=True)
    h = X + o.permute(1, 0, 2).reshape(Tn, Hq * hd) @ T_(lw["w_o"]).T
    u2 = Fn.rms_norm(h, (d,), weight=T_(lw["ffn_norm"]), eps=w.eps)
    gu = u2 @ T_(lw["w_gu"]).T
    return (h + (Fn.silu(gu[:, :F]) * gu[:, F:]) @ T_(lw["w_down"]).T).numpy()


@pytest.mark.parametrize("Hq,Hkv,gain", [(4, 2, "ones"), (4, 4, "random"), (6, 2, "random")])
def test_decoder_layer_matches_torch_composition(Hq, Hkv, gain):
    w = si.tiny(Hq=Hq, Hkv=Hkv, norm_gain=gain, L=2, n=1, Ls=1, anchors=[0, 1])
    W = si.nest_weights(si.weights_numpy_f32(si.make_weights(w)), w)
    # larger activations than the 0.02 init so attention is not uniform
    X = rng.standard_normal((9, w.d)).astype(np.float32)
    lw = W["layers"][0]
    ref = _torch_layer(w, lw, X)
    s = M._Shape(w)
    kv = M.KVCache(w.max_ctx, w.Hkv, w.hd, False)
    steps = np.stack([M.layer_step(s, lw, X[p], p, kv) for p in range(9)])
    np.testing.assert_allclose(steps, ref, rtol=1e-4, atol=1e-5)
    kv2 = M.KVCache(w.max_ctx, w.Hkv, w.hd, False)
    rows = M.layer_rows(s, lw, X, 0, kv2)
    np.testing.assert_allclose(rows, steps, rtol=1e-5, atol=1e-6)
    assert np.array_equal(kv.K[:9], kv2.K[:9]) and np.array_equal(kv.V[:9], kv2.V[:9])


def test_kv_length_assertion_guards_append_order():
    w = si.tiny()
    W = si.nest_weights(si.weights_numpy_f32(si.make_weights(w)), w)
    s = M._Shape(w)
    kv = M.KVCache(w.max_ctx, w.Hkv, w.hd, False)
    h = np.zeros(w.d, np.float32) + 0.1
    M.layer_step(s, W["layers"][0], h, 0, kv)
    with pytest.raises(AssertionError):
        M.layer_step(s, W["layers"][0], h, 2, kv)


def test_matrix_layer_equals_row_layer():
    w = si.tiny(Hq=4, Hkv=2, norm_gain="random", L=2, n=1, Ls=1, anchors=[0, 1], dtype="bf16")
    W = si.nest_weights(si.weights_numpy_f32(si.make_weights(w)), w)
    s = M._Shape(w)
    X = rng.standard_normal((7, w.d)).astype(np.float32)
    kv1 = M.KVCache(w.max_ctx, w.Hkv, w.hd, True)
    kv2 = M.KVCache(w.max_ctx, w.Hkv, w.hd, True)
    # a committed prefix of 3 positions, then 7 rows
    pre = rng.standard_normal((3, w.d)).astype(np.float32)
    M.layer_rows(s, W["layers"][0], pre, 0, kv1)
    M.layer_rows(s, W["layers"][0], pre, 0, kv2)
    a = M.layer_rows(s, W["layers"][0], X, 3, kv1)
    b = M.layer_matrix(s, W["layers"][0], X, 3, kv2)
    np.testing.assert_allclose(a, b, rtol=1e-5, atol=1e-6)


def test_matrix_prefill_gives_same_spd_run():
    from oracle import SPDOracle
    w = si.tiny(L=4, n=2, G=10, P=9, seed=17)
    W = si.nest_weights(si.weights_numpy_f32(si.make_weights(w)), w)
    prompt = si.make_prompt(w)
    a = SPDOracle(w, W)
    ta, la = a.run(prompt, w.G)
    b = SPDOracle(w, W)
    b.prefill(prompt, matrix=True)
    while b.emitted < w.G:
        b.cycle()
    assert b.tokens[: w.P + w.G] == ta
    assert [l["kv_len"] for l in b.logs] == [l["kv_len"] for l in la]


def test_ar_continue_matches_ar_greedy():
    from oracle import SPDOracle, ar_greedy
    from oracle.spd import ar_continue
    w = si.tiny(L=4, n=2, G=10, P=6, seed=18)
    W = si.nest_weights(si.weights_numpy_f32(si.make_weights(w)), w)
    prompt = si.make_prompt(w)
    ref, _ = ar_greedy(w, W, prompt, 8)
    o = SPDOracle(w, W)
    o.prefill(prompt, matrix=True)
    assert ar_continue(o, 7) == ref


def test_matrix_forward_all_rows_and_logits_rows_equal_token_forward():
    """The matrix forward over a whole sequence gives every position's final
    hidden state, anchors and logits of the row-at-a-time forward."""
    from oracle.model import Target
    w = si.tiny(L=4, n=2, P=11, seed=19, dtype="bf16", norm_gain="random")
    W = si.nest_weights(si.weights_numpy_f32(si.make_weights(w)), w)
    toks = [int(t) for t in si.make_prompt(w)]
    a, b = Target(w, W), Target(w, W)
    rows, taps_a = [], []
    for p, t in enumerate(toks):
        h, tp = a.forward_token(t, p)
        rows.append(h)
        taps_a.append(tp)
    H, taps_b = b.prefill_matrix(toks, all_rows=True)
    np.testing.assert_allclose(H, np.stack(rows), rtol=1e-4, atol=1e-5)
    for p in range(len(toks)):
        for x, y in zip(taps_a[p], taps_b[p]):
            np.testing.assert_allclose(x, y, rtol=1e-4, atol=1e-5)
    LG = b.logits_rows(H)
    for p in range(len(toks)):
        np.testing.assert_allclose(LG[p], a.logits(rows[p]), rtol=1e-4, atol=1e-5)
        assert int(np.argmax(LG[p])) == int(np.argmax(a.logits(rows[p])))


def test_feature_rows_equals_feature():
    from oracle.model import PDM
    w = si.tiny(L=8, n=4, anchors=[0, 2, 5, 8], seed=20)
    W = si.nest_weights(si.weights_numpy_f32(si.make_weights(w)), w)
    pdm = PDM(w, W)
    taps = [[rng.standard_normal(w.d).astype(np.float32) for _ in w.anchors] for _ in range(5)]
    for k in range(w.n + 1):
        a = np.stack([pdm.feature(t, k) for t in taps])
        np.testing.assert_allclose(pdm.feature_rows(taps, k), a, rtol=1e-5, atol=1e-6)


def test_rope_tables_equal_rope_cos_sin_exactly():
    from oracle.layers import rope_tables
    pos = np.arange(0, 5000, 7)
    c, s_ = rope_tables(pos, 128, 10000.0)
    for r, p in enumerate(pos):
        cp, sp = Lr.rope_cos_sin(int(p), 128, 10000.0)
        assert np.array_equal(c[r], cp) and np.array_equal(s_[r], sp), p
