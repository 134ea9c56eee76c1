"""Race check of the two-stream schedule: overlapped == serialized, bit for bit.

The draft module reads only the state from before the stage step ([PL] §3.3;
[TW] §5: drafting starts from the input state of the pipeline step, so it can
run beside the step).  The engine relies on that: the draft stream runs
beside the stage stream and the next cycle's entry joins them.  A missing
event edge, or a kernel that reads state the other stream is writing, makes
the overlapped run differ from the one where the draft chain runs alone on
the stage stream ahead of the stage step (SPD_LAUNCH_SERIALIZED).  Both runs
use graph launch and enqueue a whole generation before the first wait, so
nothing but the event edges orders the two streams.  Draft trees are
included: there the draft stream's finalisation writes the next entry's
candidates while the stage stream's verification prunes the tree.  Compared: every cycle
record, the token sequence, the last verification's logits, the last draft
logits, the anchors of the last in-flight tokens and every target layer's
KV cache.
"""
import numpy as np
import pytest

import seeded_inputs as si
from oracle import ar_greedy
from tests.gpu_common import gpu_workload_tiny

pytestmark = pytest.mark.gpu


def _generation(eng, w, first):
    eng.rollback(w.P, first)
    buf = eng.enqueue(eng.cycles_needed)
    eng.sync()
    recs = eng.records_of(buf)
    recs = recs[(recs["flags"] & 8) == 0].copy()
    recs["cycle"] -= recs["cycle"][0]  # the record counter runs on across generations
    last = recs[-1]
    t, a = int(last["t"]), int(last["occupancy"])
    state = dict(
        recs=recs.tobytes(),
        toks=eng.tokens(0, w.P + w.G),
        logits=eng.logits().tobytes(),
        pdm_logits=eng.pdm_logits().tobytes(),
        anchors=[eng.anchors(p).tobytes() for p in range(t - a + 1, t + 1)],
        kv=[(eng.kv(l, "k").tobytes(), eng.kv(l, "v").tobytes()) for l in range(w.L)],
    )
    return state, len(recs)


def _compare(w, T, uni=None, ref=None, p=None, tree=None):
    from pipelined_draft_verify_amd import SPDEngine

    eng = SPDEngine(w, T)
    if uni is not None:
        eng.set_uniforms(uni)
    if ref is not None and tree is not None:
        eng.set_tree_forced(ref, *tree)
    elif ref is not None:
        eng.set_forced(ref, p)
    first = int(eng.prefill(si.make_prompt(w)))
    # cycle count of this generation, from a first (overlapped) run
    eng.set_launch_mode(True)
    recs = eng.run(batch=64)
    eng.cycles_needed = len(recs) + 4
    out = {}
    for serial in (False, True, False):
        eng.set_launch_mode(True, serialized=serial)
        st, ncyc = _generation(eng, w, first)
        out.setdefault(serial, []).append(st)
    eng.close()
    a0, a1, b = out[False][0], out[False][1], out[True][0]
    for key in a0:
        assert a0[key] == a1[key], f"overlapped runs differ in {key}"
        assert a0[key] == b[key], f"overlapped and serialized runs differ in {key}"
    return ncyc


SMALL = {
    "tiny_fp32_natural": None,
    "bf16_n8_forced": dict(dtype="bf16", L=8, n=8, Ls=1, anchors=[0, 3, 8], G=30, seed=71),
    "bf16_split_1232_forced": dict(dtype="bf16", L=8, n=4, split=(1, 2, 3, 2), Ls=2, anchors=[0, 1, 3, 6, 8],
                                   G=30, seed=72),
    "bf16_sample_dense": dict(dtype="bf16", mode="sample", L=6, n=3, Hq=8, Hkv=2, F=768, V=500,
                              anchors=[0, 2, 5], Ls=2, G=30, seed=73),
    "f32_sample_topk12": dict(dtype="f32", mode="sample", top_k=12, V=40, G=30, seed=74),
    "bf16_hybrid_forced": dict(dtype="bf16", L=8, n=4, Ls=2, anchors=[0, 2, 4, 8], attn_period=4, G=30,
                               seed=75),
    # draft trees: the draft stream's finalisation writes the candidates while
    # the stage stream's verification prunes the tree
    "bf16_tree_w4_forced": dict(dtype="bf16", L=8, n=4, Hq=8, Hkv=2, F=768, V=500, anchors=[0, 2, 4, 8], Ls=2,
                                width=4, G=30, seed=76),
    "f32_tree_w3_natural": dict(dtype="f32", L=4, n=4, anchors=[0, 1, 2, 3, 4], width=3, G=30, seed=77),
}


@pytest.mark.parametrize("name", sorted(SMALL))
def test_overlapped_equals_serialized_small(name):
    kw = SMALL[name]
    w = si.workload("tiny_fp32", G=40) if kw is None else gpu_workload_tiny(**kw)
    T = si.make_weights(w, "cpu")
    uni = si.make_uniforms(w)
    ref = p = tree = None
    if kw is not None and w.mode == "greedy" and not name.endswith("natural"):
        W = si.nest_weights(si.weights_numpy_f32(T), w)
        ref, _ = ar_greedy(w, W, si.make_prompt(w), w.G)
        p = 0.6
        tree = (0.3, 0.8) if w.width > 1 else None
    ncyc = _compare(w, {k: v.to("cuda:0") for k, v in T.items()}, uni=uni, ref=ref, p=p, tree=tree)
    print(f"{name}: {ncyc} cycles bit-identical overlapped and serialized")


def test_overlapped_equals_serialized_full_size_4b_n8():
    """The headline workload at full size: 4B-class shapes, n = 8, forced 0.8."""
    import torch
    from pipelined_draft_verify_amd import SPDEngine

    w = si.workload("4b_n8")
    T = si.make_weights(w, "cuda:0")
    uni = si.make_uniforms(w)
    eng = SPDEngine(w, T)
    eng.set_uniforms(uni)
    prompt = si.make_prompt(w)
    first = int(eng.prefill(prompt))
    ar = eng.generate_ar(w.G - 1)
    ref = [int(x) for x in prompt] + [first] + [int(x) for x in ar]
    eng.close()
    del eng
    ncyc = _compare(w, T, uni=uni, ref=ref, p=w.p_accept)
    print(f"4b_n8: {ncyc} cycles bit-identical overlapped and serialized")
    del T
    torch.cuda.empty_cache()


def test_overlapped_equals_serialized_full_size_tree():
    """The width-4 draft tree on the 4B-class shapes (n = 8, forced tree policy)."""
    import torch
    from pipelined_draft_verify_amd import SPDEngine

    w = si.workload("4b_tree4_n8")
    T = si.make_weights(w, "cuda:0")
    uni = si.make_uniforms(w)
    eng = SPDEngine(w, T)
    eng.set_uniforms(uni)
    prompt = si.make_prompt(w)
    first = int(eng.prefill(prompt))
    ar = eng.generate_ar(w.G - 1)
    ref = [int(x) for x in prompt] + [first] + [int(x) for x in ar]
    eng.close()
    del eng
    ncyc = _compare(w, T, uni=uni, ref=ref, tree=(w.p_accept, w.p_tree))
    print(f"4b_tree4_n8: {ncyc} cycles bit-identical overlapped and serialized")
    del T
    torch.cuda.empty_cache()
