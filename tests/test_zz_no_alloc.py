"""The allocation-free init (spd_init_static_scratch) against spd_init.

The same workload runs once on an engine whose scratch is carved from its
workspace (spd_init) and once on an engine whose scratch is the library's
static device array (spd_init_static_scratch); records, tokens, logits, draft
logits, anchors and KV caches must be bit-identical.  Static-scratch engines
in a row, the second with a smaller input, so that it starts from the first
one's leftover scratch contents, and a third with a small draft tree.
"""
import numpy as np
import pytest

import seeded_inputs as si
from oracle import ar_greedy
from tests.gpu_common import gpu_workload_tiny

pytestmark = pytest.mark.gpu


def _run(w, T, static, uni, ref, p, tree=None):
    from pipelined_draft_verify_amd import SPDEngine

    eng = SPDEngine(w, T, static_scratch=static)
    eng.set_uniforms(uni)
    if ref is not None and tree is not None:
        eng.set_tree_forced(ref, *tree)
    elif ref is not None:
        eng.set_forced(ref, p)
    eng.prefill(si.make_prompt(w))
    recs = eng.run(batch=128)
    last = recs[-1]
    t, a = int(last["t"]), int(last["occupancy"])
    out = dict(ws=eng.ws_bytes, recs=recs.tobytes(), toks=eng.tokens(0, w.P + w.G),
               logits=eng.logits().tobytes(), pdm_logits=eng.pdm_logits().tobytes(),
               anchors=[eng.anchors(q).tobytes() for q in range(t - a + 1, t + 1)],
               # committed positions only: the cache beyond a layer's length is never
               # written and holds whatever the two engines' buffers held before
               kv=[(eng.kv(l, "k")[: int(last["kv_len"][l])].tobytes(),
                    eng.kv(l, "v")[: int(last["kv_len"][l])].tobytes()) for l in sorted({0, w.L - 1})])
    eng.close()
    return out


def _check(w, T, uni, ref=None, p=None, tree=None):
    a = _run(w, T, False, uni, ref, p, tree)
    b = _run(w, T, True, uni, ref, p, tree)
    assert b["ws"] < a["ws"]  # the static engine's workspace holds no scratch
    for k in a:
        if k != "ws":
            assert a[k] == b[k], f"{w.name}: {k} differs between spd_init and spd_init_static_scratch"
    return len(np.frombuffer(a["recs"], dtype=np.uint8))


def test_static_scratch_matches_spd_init_two_calls():
    import torch

    # first call: the 4B-class n=8 workload at full size (forced acceptance 0.8)
    from pipelined_draft_verify_amd import SPDEngine
    w = si.workload("4b_n8")
    T = si.make_weights(w, "cuda:0")
    uni = si.make_uniforms(w)
    eng = SPDEngine(w, T)
    prompt = si.make_prompt(w)
    first = int(eng.prefill(prompt))
    ref = [int(x) for x in prompt] + [first] + [int(x) for x in eng.generate_ar(w.G - 1)]
    eng.close()
    _check(w, T, uni, ref, w.p_accept)
    del T
    torch.cuda.empty_cache()
    # second call, smaller input: a small bf16 model with dense T=1 sampling
    w2 = gpu_workload_tiny(dtype="bf16", mode="sample", L=6, n=3, Hq=8, Hkv=2, F=768, V=500, anchors=[0, 2, 5],
                           Ls=2, G=24, seed=81)
    T2 = {k: v.to("cuda:0") for k, v in si.make_weights(w2, "cpu").items()}
    _check(w2, T2, si.make_uniforms(w2))
    # third call: a small bf16 draft tree (its per-leaf scan partials live in the scratch too)
    w3 = gpu_workload_tiny(dtype="bf16", L=8, n=4, Hq=8, Hkv=2, F=768, V=500, anchors=[0, 2, 4, 8], Ls=2,
                           width=4, G=24, seed=82)
    T3c = si.make_weights(w3, "cpu")
    W3 = si.nest_weights(si.weights_numpy_f32(T3c), w3)
    ref3, _ = ar_greedy(w3, W3, si.make_prompt(w3), w3.G)
    T3 = {k: v.to("cuda:0") for k, v in T3c.items()}
    _check(w3, T3, si.make_uniforms(w3), ref=ref3, tree=(0.3, 0.8))
