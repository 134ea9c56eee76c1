"""GPU parity on the degenerate cases and the size limits of the method.

  * one stage (n = 1): every token exits in the cycle it enters, verifying the
    draft made in that same cycle; with the most draft-module layers
    (SPD_MAX_PDM_LAYERS = 8) and with bf16;
  * the most anchors (SPD_MAX_ANCHORS = 8, one fusion matrix each) and the
    most target layers and stages (SPD_MAX_LAYERS = 64, SPD_MAX_STAGES = 16);
  * GEMV inputs longer than 4096 elements, which the stage GEMV stages in two
    passes instead of from registers (bf16 and fp32);
  * a generation of one token (prefill only: the cycles that follow are
    idle) and of two (one verification);
  * an empty prompt is refused;
  * the longest context (max_ctx = 32768: 128 attention splits): natural and
    forced drafts emit exactly the GPU's own autoregressive greedy decode (a
    property that holds at any size), and the oracle's forward over the
    final ~32k-token sequence (matrix form, about a minute on the host) checks
    the first token and every verification's target token, and the last
    verification's logits;
  * the largest vocabulary (SPD_MAX_VOCAB = 2^20 ids) in sample mode, dense
    and with top-64 truncation, and the smallest (2 and 3 ids).
Every run through the oracle must agree cycle by cycle as in the other
small-workload parity tests.
"""
import numpy as np
import pytest

import seeded_inputs as si
from oracle import ar_greedy
from tests.gpu_common import compare_logs, gpu_workload_tiny, run_gpu
from tests.test_gpu_parity_small import _inputs, _oracle

pytestmark = pytest.mark.gpu

IDLE = 8

EDGE = {
    "n1_Ls4_bf16": dict(dtype="bf16", L=4, n=1, Ls=4, anchors=[0, 1, 2, 3, 4], G=16, p=0.6, seed=51),
    "n1_Ls8_f32": dict(L=8, n=1, Ls=8, anchors=[0, 4, 8], G=14, p=0.6, seed=52),
    "m8_anchors_bf16": dict(dtype="bf16", L=8, n=2, Ls=2, anchors=[0, 1, 2, 3, 4, 5, 6, 7], p=0.6, seed=53),
    "L64_n16_f32": dict(L=64, n=16, Ls=4, anchors=[0, 16, 32, 48, 64], G=40, p=0.7, seed=54),
    # GEMV inputs longer than the register-staged 4096 elements (model width
    # and query heads x head dim 4608): the two-pass staging path
    "d4608_bf16": dict(dtype="bf16", L=4, n=2, Ls=1, d=4608, Hq=72, Hkv=9, F=512, anchors=[0, 2, 4], p=0.6,
                       seed=55),
    "d4352_f32": dict(L=4, n=2, Ls=1, d=4352, F=512, anchors=[0, 2, 4], p=0.6, seed=56),
}


@pytest.mark.parametrize("name", sorted(EDGE))
def test_edge_shape_matches_oracle(name):
    kw = dict(EDGE[name])
    p = kw.pop("p")
    w = gpu_workload_tiny(**kw)
    T, W, prompt, uni = _inputs(w)
    ref, _ = ar_greedy(w, W, prompt, w.G)
    eng, first, recs, toks = run_gpu(w, T, prompt, uni=uni, ref=ref, p_accept=p)
    eng.close()
    o, otoks, ologs = _oracle(w, W, prompt, uni, recs, first, ref=ref, p=p)
    assert not o.dec.mismatch, o.dec.mismatch
    assert len(o.dec.adopted) <= 2, o.dec.adopted
    assert toks == otoks == ref
    compare_logs(recs, ologs, w.L)
    acc = recs["accepted"][recs["exit_pos"] >= 0]
    assert (acc == 1).any() and (acc == 0).any()
    if w.n == 1:
        assert len(recs) == w.G - 1  # one token per cycle
        assert (recs["occupancy"] == 1).all() and (recs["exit_pos"] == recs["t"]).all()


@pytest.mark.parametrize("G", [1, 2])
def test_one_and_two_token_generations(G):
    w = gpu_workload_tiny(G=G, seed=55 + G)
    T, W, prompt, uni = _inputs(w)
    ref, _ = ar_greedy(w, W, prompt, w.G)
    from pipelined_draft_verify_amd import SPDEngine

    eng = SPDEngine(w, {k: v.to("cuda:0") for k, v in T.items()})
    eng.set_uniforms(uni)
    first = eng.prefill(prompt)
    recs = eng.run()
    toks = eng.tokens(w.P, w.G)
    eng.close()
    assert [first] + toks[1:] == ref[w.P:] == toks
    assert len(recs) == (0 if G == 1 else w.n)
    if G == 2:
        assert (recs["exit_pos"] >= 0).sum() == 1


def test_empty_prompt_is_refused():
    w = gpu_workload_tiny(seed=58)
    T, W, prompt, uni = _inputs(w)
    from pipelined_draft_verify_amd import SPDEngine, SPDError

    eng = SPDEngine(w, {k: v.to("cuda:0") for k, v in T.items()})
    with pytest.raises(SPDError):
        eng.prefill([])
    first = eng.prefill(prompt)  # still usable afterwards
    eng.run()
    assert eng.tokens(w.P, 1) == [first]
    eng.close()


def test_longest_context_is_lossless():
    G, n = 12, 2
    P = 32768 - G - n - 8  # max_ctx = P + G + n + 8 = 32768, the largest accepted
    w = gpu_workload_tiny(dtype="bf16", L=2, n=n, Ls=1, anchors=[0, 1, 2], Hq=4, Hkv=1, P=P, G=G, seed=59)
    assert w.max_ctx == 32768
    T = si.make_weights(w, "cuda:0")
    prompt = si.make_prompt(w)
    from pipelined_draft_verify_amd import SPDEngine

    eng = SPDEngine(w, T)
    eng.set_uniforms(si.make_uniforms(w))
    first = eng.prefill(prompt)
    ar = eng.generate_ar(G - 1)
    for p in (None, 0.5):
        eng.rollback(P, first)
        if p is not None:
            eng.set_forced(list(prompt) + [first] + ar, p)
        recs = eng.run()
        assert eng.tokens(P, G) == [first] + ar, p
        ex = recs[recs["exit_pos"] >= 0]
        assert len(ex) == G - 1 and int(ex["exit_pos"][-1]) == P + G - 2
        assert int(recs["t"].max()) < w.max_ctx
    toks = [int(x) for x in eng.tokens(0, P + G)]
    last_logits = eng.logits()
    eng.close()
    # the oracle's target forward over the final sequence (positions 0 .. P+G-2)
    from oracle.model import Target
    from oracle.spd import Decisions
    from tests.full_size import rel_l2

    W = si.nest_weights(si.weights_numpy_f32(T), w)
    del T
    tgt = Target(w, W)
    H, _ = tgt.prefill_matrix(toks[: P + G - 1], all_rows=True)
    LG = tgt.logits_rows(H[P - 1:])
    del H
    teacher = {("y", j): toks[j + 1] for j in range(P - 1, P + G - 1)}
    dec = Decisions(teacher, 0.05)
    for j in range(P - 1, P + G - 1):
        dec.argmax(("y", j), LG[j - (P - 1)])
    print(f"longest context: {G} target tokens checked against the oracle, {len(dec.adopted)} near-ties adopted")
    assert not dec.mismatch, dec.mismatch[:5]
    assert len(dec.adopted) <= 2
    err = rel_l2(last_logits, LG[-1])
    print(f"longest context: last verification logits rel-L2 {err:.3g}")
    assert err <= 2e-2


@pytest.mark.parametrize("top_k", [0, 64])
def test_sampling_at_the_largest_vocabulary(top_k):
    """V = SPD_MAX_VOCAB = 2^20: 4096 sampler blocks in 64 superblocks (dense),
    or the top-64 selection over 2^20 ids.  Near-uniform random-init
    distributions put ~1e-6 of the mass on each id, so differing draws may
    land on a neighbouring id; each must lie within the sampling tolerance."""
    from tests.test_gpu_parity_small import STOL, TOL
    from tests.gpu_common import teacher_of
    from oracle import SPDOracle

    w = gpu_workload_tiny(mode="sample", temperature=1.0, V=1 << 20, L=2, n=2, Ls=1, anchors=[0, 1, 2], G=10,
                          top_k=top_k, seed=60 + top_k)
    T, W, prompt, uni = _inputs(w)
    eng, first, recs, toks = run_gpu(w, T, prompt, uni=uni)
    eng.close()
    o = SPDOracle(w, W, uniforms=uni, teacher=teacher_of(recs, first), tol=TOL[w.dtype], sample_tol=STOL[w.dtype])
    otoks, ologs = o.run(prompt, w.G)
    assert not o.dec.mismatch, o.dec.mismatch
    assert toks == otoks
    compare_logs(recs, ologs, w.L)


@pytest.mark.parametrize("V,mode,top_k", [(2, "greedy", 0), (3, "sample", 0), (3, "sample", 2)])
def test_smallest_vocabularies(V, mode, top_k):
    """V = 2 and 3: one partial block of the sampler and of the argmax, a
    top-k list longer than half the vocabulary."""
    from tests.test_gpu_parity_small import STOL, TOL
    from tests.gpu_common import teacher_of
    from oracle import SPDOracle

    kw = dict(V=V, L=4, n=2, G=16, seed=70 + V + top_k)
    if mode == "sample":
        kw.update(mode="sample", temperature=1.0, top_k=top_k)
    w = gpu_workload_tiny(**kw)
    T, W, prompt, uni = _inputs(w)
    if mode == "sample":
        eng, first, recs, toks = run_gpu(w, T, prompt, uni=uni)
        eng.close()
        o = SPDOracle(w, W, uniforms=uni, teacher=teacher_of(recs, first), tol=TOL[w.dtype],
                      sample_tol=STOL[w.dtype])
        otoks, ologs = o.run(prompt, w.G)
    else:
        ref, _ = ar_greedy(w, W, prompt, w.G)
        eng, first, recs, toks = run_gpu(w, T, prompt, uni=uni, ref=ref, p_accept=0.5)
        eng.close()
        o, otoks, ologs = _oracle(w, W, prompt, uni, recs, first, ref=ref, p=0.5)
    assert not o.dec.mismatch, o.dec.mismatch
    assert toks == otoks
    assert all(0 <= t < V for t in toks)
    compare_logs(recs, ologs, w.L)
