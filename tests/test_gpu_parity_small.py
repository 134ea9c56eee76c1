"""GPU parity on small workloads the oracle runs completely (seconds).

The HIP path and the oracle run the same seeded weights, prompt, uniforms and
draft policy.  Token ids, drafts, accept decisions, KV lengths, occupancy and
the draft module's committed length must agree bit for bit every cycle.
Where floating point decides an integer (an argmax), a near-tie is the only
allowed difference: the oracle adopts the GPU's choice when that choice's
logit is within the tolerance of the oracle's maximum (1e-4 in fp32,
0.05 in bf16), and the test counts such adoptions (expected: none or a few).
Hidden states, anchors and logits must match within rel-L2 1e-4 (fp32) and
2e-2 (bf16).
"""
import numpy as np
import pytest

import seeded_inputs as si
from oracle import ForcedPolicy, SPDOracle, ar_greedy
from tests.gpu_common import compare_logs, gpu_workload_tiny, rel_l2, run_gpu, run_gpu_with_sets, teacher_of

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 0.05}
RTOL = {"f32": 1e-4, "bf16": 2e-2}


def _inputs(w):
    T = si.make_weights(w, "cpu")
    W = si.nest_weights(si.weights_numpy_f32(T), w)
    return T, W, si.make_prompt(w), si.make_uniforms(w)


def _oracle(w, W, prompt, uni, recs, first, ref=None, p=None):
    pol = ForcedPolicy(ref, p, uni, w.V) if ref is not None else None
    o = SPDOracle(w, W, policy=pol, uniforms=uni, teacher=teacher_of(recs, first), tol=TOL[w.dtype])
    toks, logs = o.run(prompt, w.G)
    return o, toks, logs


def test_tiny_fp32_workload_matches_oracle():
    """The tiny fp32 workload (L=8, d=256, n=4, natural drafts), all 64 tokens."""
    w = si.workload("tiny_fp32")
    T, W, prompt, uni = _inputs(w)
    eng, first, recs, toks = run_gpu(w, T, prompt)
    eng.close()
    o, otoks, ologs = _oracle(w, W, prompt, uni, recs, first)
    assert not o.dec.mismatch
    assert len(o.dec.adopted) == 0, o.dec.adopted
    assert toks == otoks
    compare_logs(recs, ologs, w.L)


VARIANTS = {
    "gqa_f32_forced": dict(dtype="f32", p=0.6),
    "bf16_gqa_forced": dict(dtype="bf16", L=6, n=3, Hq=8, Hkv=2, F=768, V=500, anchors=[0, 2, 5], Ls=2, p=0.5,
                            seed=32),
    "deep_n8": dict(L=8, n=8, Ls=1, anchors=[0, 3, 8], G=20, p=0.7, seed=33),
    "hd128_bf16": dict(dtype="bf16", Hq=2, Hkv=1, hd=128, F=512, V=700, p=0.8, seed=34, norm_gain="random"),
    "mha_n4_long_prompt": dict(L=4, n=4, Hq=4, Hkv=4, anchors=[0, 1, 2, 3, 4], P=300, G=16, p=0.5, seed=35),
    "g5_gqa_bf16": dict(dtype="bf16", d=256, Hq=20, Hkv=4, hd=64, F=512, V=1000, L=4, n=4, Ls=1,
                        anchors=[0, 2, 3], P=40, G=20, p=0.8, seed=36),
    # n = 16: up to 17 draft-module rows (two row tiles), all in one fusion pattern
    "n16_one_anchor_bf16": dict(dtype="bf16", L=16, n=16, Ls=1, anchors=[0], G=40, p=0.7, seed=43),
    "n16_one_anchor_f32": dict(dtype="f32", L=16, n=16, Ls=1, anchors=[0], G=40, p=0.7, seed=44),
    # post-step schedule: the draft module reads the features after the stage step
    "post_f32_forced": dict(dtype="f32", p=0.6, seed=37, schedule="post"),
    "post_bf16_gqa_forced": dict(dtype="bf16", L=6, n=3, Hq=8, Hkv=2, F=768, V=500, anchors=[0, 2, 5], Ls=2,
                                 p=0.5, seed=38, schedule="post"),
    "post_deep_n8": dict(L=8, n=8, Ls=1, anchors=[0, 3, 8], G=20, p=0.7, seed=39, schedule="post"),
    # non-uniform stage splits: sub-steps where some stages have no layer left
    "split_132_f32": dict(L=6, n=3, split=(1, 3, 2), Ls=2, anchors=[0, 1, 4, 6], p=0.6, seed=57),
    "split_3122_bf16": dict(dtype="bf16", L=8, n=4, split=(3, 1, 2, 2), Ls=3, anchors=[0, 2, 4, 6, 7], Hq=8,
                            Hkv=2, F=512, p=0.6, seed=58),
    "split_213_post_f32": dict(L=6, n=3, split=(2, 1, 3), Ls=3, anchors=[0, 1, 4, 6], p=0.6, seed=59,
                               schedule="post"),
    "split_35_hybrid_bf16": dict(dtype="bf16", L=8, n=2, split=(3, 5), Ls=2, anchors=[0, 3, 8], attn_period=4,
                                 p=0.6, seed=60),
}


@pytest.mark.parametrize("name", sorted(VARIANTS))
def test_variant_matches_oracle(name):
    kw = dict(VARIANTS[name])
    p = kw.pop("p")
    w = gpu_workload_tiny(**kw)
    T, W, prompt, uni = _inputs(w)
    ref, _ = ar_greedy(w, W, prompt, w.G)
    eng, first, recs, toks = run_gpu(w, T, prompt, uni=uni, ref=ref, p_accept=p)
    eng.close()
    o, otoks, ologs = _oracle(w, W, prompt, uni, recs, first, ref=ref, p=p)
    assert not o.dec.mismatch, o.dec.mismatch
    assert len(o.dec.adopted) <= 2, o.dec.adopted
    assert toks == otoks
    compare_logs(recs, ologs, w.L)
    # the acceptance structure is exercised
    acc = recs["accepted"]
    assert (acc == 1).any() and (acc == 0).any()


# temperature sampling with rejection-sampling verification
SAMPLE_VARIANTS = {
    "f32_T1": dict(dtype="f32", temperature=1.0, seed=40),
    "split_132_f32_T1": dict(dtype="f32", temperature=1.0, L=6, n=3, split=(1, 3, 2), Ls=2, anchors=[0, 1, 4, 6],
                             seed=61),
    "f32_T0.3": dict(dtype="f32", temperature=0.3, seed=40),
    "bf16_n4_T0.3": dict(dtype="bf16", temperature=0.3, L=4, n=4, anchors=[0, 1, 2, 3, 4], G=30, seed=41),
    "bf16_gqa_T0.5": dict(dtype="bf16", temperature=0.5, L=6, n=3, Hq=8, Hkv=2, F=768, V=500,
                          anchors=[0, 2, 5], Ls=2, seed=42),
    # odd vocabulary over several superblocks of the sampler's block sums:
    # tail blocks, unaligned draft-weight slots, multi-level search
    "f32_V20001_T1": dict(dtype="f32", temperature=1.0, V=20001, seed=43),
    "f32_post_T1": dict(dtype="f32", temperature=1.0, seed=46, schedule="post"),
    # top-k truncation of P and Q (the pages' evaluation decodes with top-k 50)
    "f32_topk50_T1": dict(dtype="f32", temperature=1.0, seed=47, top_k=50),
    "bf16_gqa_topk50_T0.7": dict(dtype="bf16", temperature=0.7, L=6, n=3, Hq=8, Hkv=2, F=768, V=500,
                                 anchors=[0, 2, 5], Ls=2, seed=48, top_k=50),
    "f32_post_topk12_V24_T1": dict(dtype="f32", temperature=1.0, seed=49, top_k=12, V=24, schedule="post"),
    # k = 64 over an odd vocabulary spanning many blocks: two unrelated top-64
    # sets out of 20001 ids hardly overlap, so drafts are (almost) never accepted
    "f32_V20001_topk64_T1": dict(dtype="f32", temperature=1.0, V=20001, seed=50, top_k=64, need_accepts=False),
}
# a differing draw is a near-tie only if the threshold lies this close (as a
# fraction of the total mass, or of Q(x) for the accept test) to its boundary
STOL = {"f32": 1e-5, "bf16": 2e-4}


@pytest.mark.parametrize("name", sorted(SAMPLE_VARIANTS))
def test_sampling_matches_oracle(name):
    """Draws from Q, accept tests u*Q(x) < P(x) and residual redraws from
    max(0, P - Q) use the same seeded uniforms on both sides; every integer
    of every cycle must agree."""
    kw = dict(SAMPLE_VARIANTS[name])
    need_accepts = kw.pop("need_accepts", True)
    w = gpu_workload_tiny(mode="sample", **kw)
    T, W, prompt, uni = _inputs(w)
    sets = None
    if w.top_k:
        # top-k: the GPU's kept sets (from its logits) must be valid top-k
        # choices of the oracle's logits, and the draws are retaken on them
        eng, first, recs, toks, sets = run_gpu_with_sets(w, T, prompt, uni)
    else:
        eng, first, recs, toks = run_gpu(w, T, prompt, uni=uni)
    eng.close()
    o = SPDOracle(w, W, uniforms=uni, teacher=teacher_of(recs, first, sets), tol=TOL[w.dtype],
                  sample_tol=STOL[w.dtype])
    otoks, ologs = o.run(prompt, w.G)
    print(name, "adopted", o.dec.adopted)
    assert not o.dec.mismatch, o.dec.mismatch
    assert len(o.dec.adopted) <= 2, o.dec.adopted
    assert toks == otoks
    compare_logs(recs, ologs, w.L)
    acc = recs["accepted"][recs["exit_pos"] >= 0]
    assert (acc == 0).any()
    assert (acc == 1).any() or not need_accepts


@pytest.mark.parametrize("split", [(), (1, 2, 3, 2)])
def test_eager_and_graph_launch_agree(split):
    """Host-launched and graph-replayed cycles give bit-identical records and
    tokens (uniform split, and uneven stages whose sub-steps hold different
    group sets)."""
    L = sum(split) if split else 4
    w = gpu_workload_tiny(dtype="bf16", L=L, n=4, anchors=[0, 1, 2, 3, 4], G=30, seed=45, split=split)
    T, W, prompt, uni = _inputs(w)
    ref, _ = ar_greedy(w, W, prompt, w.G)
    from pipelined_draft_verify_amd import SPDEngine

    eng = SPDEngine(w, {k: v.to("cuda:0") for k, v in T.items()})
    eng.set_uniforms(uni)
    eng.set_forced(ref, 0.6)
    first = eng.prefill(prompt)
    out = {}
    for mode in (False, True, False):
        eng.rollback(w.P, first)
        eng.set_launch_mode(mode)
        recs = eng.run(batch=16)
        recs["cycle"] -= recs["cycle"][0]   # the record counter runs on across generations
        out.setdefault(mode, []).append((recs.tobytes(), eng.tokens(0, w.P + w.G)))
    eng.close()
    assert out[False][0] == out[True][0] == out[False][1]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_hidden_states_anchors_and_logits(dtype):
    """Per-cycle anchors of every in-flight token and the verification logits."""
    w = gpu_workload_tiny(dtype=dtype, L=4, n=2, G=12, seed=37)
    T, W, prompt, uni = _inputs(w)
    ref, _ = ar_greedy(w, W, prompt, w.G)
    gpu = {}

    def hook(eng, r):
        c = int(r["cycle"])
        t, a = int(r["t"]), int(r["occupancy"])
        # in-flight tokens after the stage step (the exiting one is still in its slot)
        gpu[c] = {"anchors": {p: eng.anchors(p) for p in range(t - a + 1, t + 1)}}
        if r["exit_pos"] >= 0:
            gpu[c]["logits"] = eng.logits()
        gpu[c]["pdm_logits"] = eng.pdm_logits()

    eng, first, recs, toks = run_gpu(w, T, prompt, uni=uni, ref=ref, p_accept=0.5, per_cycle_hook=hook)
    eng.close()
    pol = ForcedPolicy(ref, 0.5, uni, w.V)
    o = SPDOracle(w, W, policy=pol, uniforms=uni, teacher=teacher_of(recs, first), tol=TOL[dtype])
    seen = {"exit": 0, "pdm": 0, "anch": 0}

    def ohook(kind, info):
        c = info["cycle"]
        if kind == "exit":
            assert rel_l2(gpu[c]["logits"], info["logits"]) <= RTOL[dtype]
            seen["exit"] += 1
        elif kind == "pdm":
            assert rel_l2(gpu[c]["pdm_logits"], info["logits"]) <= RTOL[dtype]
            seen["pdm"] += 1

    o.hook = ohook
    o.prefill(prompt)
    while o.emitted < w.G:
        rec = o.cycle()
        c = rec["cycle"]
        for p, ga in gpu[c]["anchors"].items():
            taps = o.anchors.get(p)
            if taps is None:
                continue
            for i, a in enumerate(taps):
                if a is not None:
                    assert rel_l2(ga[i], a) <= RTOL[dtype], (c, p, i)
                    seen["anch"] += 1
    assert seen["exit"] > 3 and seen["pdm"] == len(recs) and seen["anch"] > 10


def test_lossless_forced_natural_and_autoregressive_agree():
    """On the GPU alone: natural drafts, forced drafts and plain AR decoding
    emit bit-identical tokens (the method is lossless for any draft policy)."""
    w = gpu_workload_tiny(dtype="bf16", L=4, n=4, anchors=[0, 1, 2, 3, 4], G=30, seed=38)
    T, W, prompt, uni = _inputs(w)
    import torch
    from pipelined_draft_verify_amd import SPDEngine

    eng = SPDEngine(w, {k: v.to("cuda:0") for k, v in T.items()})
    eng.set_uniforms(uni)
    first = eng.prefill(prompt)
    ar = eng.generate_ar(w.G - 1)
    eng.rollback(w.P, first)
    nat = eng.run()
    tok_nat = eng.tokens(w.P, w.G)
    ref = list(prompt) + [first] + ar
    for p in (0.0, 0.5, 1.0):
        eng.rollback(w.P, first)
        eng.set_forced(ref, p)
        recs = eng.run()
        assert eng.tokens(w.P, w.G) == [first] + ar, p
        if p == 1.0:
            assert (recs["accepted"][recs["exit_pos"] >= 0] == 1).all()
            assert len(recs) == w.n + w.G - 2
    eng.close()
    assert tok_nat == [first] + ar


@pytest.mark.parametrize("split", [(), (1, 3)])
def test_rollback_to_prefix_equals_fresh_prefill(split):
    w = gpu_workload_tiny(dtype="f32", L=4, n=2, G=16, seed=39, split=split)
    T, W, prompt, uni = _inputs(w)
    from pipelined_draft_verify_amd import SPDEngine

    eng = SPDEngine(w, {k: v.to("cuda:0") for k, v in T.items()})
    first = eng.prefill(prompt)
    eng.run()
    toks = eng.tokens(0, w.P + w.G)
    keep = w.P + 5
    eng.rollback(keep, toks[keep])
    st = eng.sync()
    assert st.emitted == keep - w.P + 1
    recs = eng.run()
    assert eng.tokens(0, w.P + w.G) == toks
    kv_a = eng.kv(1, "k")[:keep]
    eng.close()
    # a fresh engine prefilled with the kept prefix holds the same KV entries
    w2 = w.replace(P=keep)
    eng2 = SPDEngine(w2, {k: v.to("cuda:0") for k, v in T.items()})
    eng2.prefill(toks[:keep])
    kv_b = eng2.kv(1, "k")[:keep]
    eng2.close()
    np.testing.assert_allclose(kv_a, kv_b, rtol=1e-5, atol=1e-6)


def test_error_paths_from_the_host():
    w = gpu_workload_tiny()
    T, W, prompt, uni = _inputs(w)
    from pipelined_draft_verify_amd import SPDEngine, SPDError

    eng = SPDEngine(w, {k: v.to("cuda:0") for k, v in T.items()})
    with pytest.raises(SPDError):      # cycles before prefill
        eng.enqueue(1, log=False)
    with pytest.raises(SPDError):      # prompt too long for max_ctx
        eng.prefill([1] * (w.max_ctx))
    first = eng.prefill(prompt)
    with pytest.raises(SPDError):      # rollback beyond the verified prefix
        eng.rollback(w.P + 3, first)
    with pytest.raises(SPDError):      # token out of range
        eng.rollback(w.P, w.V)
    eng.run()
    eng.close()


def test_setter_refusals_from_the_host():
    """The policy, uniform-table and launch-mode calls refuse what their
    declarations exclude, and a refused call leaves the engine usable."""
    from pipelined_draft_verify_amd import SPDEngine, SPDError
    from pipelined_draft_verify_amd import _abi as A

    def einval(fn, *args):
        with pytest.raises(SPDError) as e:
            fn(*args)
        assert e.value.code == A.SPD_EINVAL

    # a chain
    w = gpu_workload_tiny(seed=61)
    T, W, prompt, uni = _inputs(w)
    ref, _ = ar_greedy(w, W, prompt, w.G)
    eng = SPDEngine(w, {k: v.to("cuda:0") for k, v in T.items()})
    einval(eng.set_forced, ref, 0.8)                 # forced drafts need the uniform table
    einval(eng.set_uniforms, uni[: w.max_ctx - 1])   # fewer positions than the context holds
    eng.set_uniforms(uni)
    einval(eng.set_forced, ref, 1.5)                 # acceptance outside [0, 1]
    einval(eng.set_tree_forced, ref, 0.3, 0.8)       # the tree policy on a chain
    einval(A.spd_set_launch_mode, eng.h, 4)          # not eager or graph
    einval(eng.prefill, list(prompt[:-1]) + [w.V])   # a prompt token outside the vocabulary
    eng.set_forced(ref, 0.8)
    first = eng.prefill(prompt)
    eng.run()
    toks = eng.tokens(w.P, w.G)
    eng.close()
    assert [first] + toks[1:] == ref[w.P:] == toks

    # a draft tree
    w = gpu_workload_tiny(L=4, n=2, width=2, seed=62)
    T, W, prompt, uni = _inputs(w)
    ref, _ = ar_greedy(w, W, prompt, w.G)
    eng = SPDEngine(w, {k: v.to("cuda:0") for k, v in T.items()})
    eng.set_uniforms(uni)
    einval(eng.set_forced, ref, 0.8)                 # a tree takes the tree policy
    einval(eng.set_tree_forced, ref, 0.9, 0.5)       # p_first above p_tree
    eng.set_tree_forced(ref, 0.3, 0.8)
    first = eng.prefill(prompt)
    eng.run()
    toks = eng.tokens(w.P, w.G)
    eng.close()
    assert [first] + toks[1:] == ref[w.P:] == toks
