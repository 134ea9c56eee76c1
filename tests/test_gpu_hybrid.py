"""GPU parity of the hybrid target (linear-attention layers between softmax layers).

The oracle computes a linear layer from its definition (weights
phi(q).phi(k_i) over the cached keys and values); the HIP path runs the
recurrent form on a per-position state ring.  The same cycle-by-cycle bar as
the other small workloads applies: every integer of every cycle equal, near
ties adopted only within the argmax tolerance.  Also on the GPU alone: the
pipeline with any draft policy emits exactly the GPU's own autoregressive
decode (through the prefill checkpoint of the linear-attention states), and
a rollback to a length whose state is no longer held is refused.
"""
import numpy as np
import pytest

import seeded_inputs as si
from oracle import SPDOracle, ar_greedy
from tests.gpu_common import compare_logs, gpu_workload_tiny, run_gpu, teacher_of
from tests.test_gpu_parity_small import STOL, TOL, _inputs, _oracle

pytestmark = pytest.mark.gpu

HYBRID = {
    # period 2 with 2 layers per stage: sub-step 0 all linear, 1 all softmax
    "f32_n2_P2": dict(L=4, n=2, Ls=1, anchors=[0, 2, 3], attn_period=2, p=0.6, seed=71),
    # period 4 with 2 layers per stage: sub-step 1 mixes linear and softmax groups
    "bf16_n4_P4_mixed": dict(dtype="bf16", L=8, n=4, Ls=2, anchors=[0, 2, 4, 6, 7], attn_period=4, G=30,
                             p=0.6, seed=72),
    "bf16_hd128_gqa": dict(dtype="bf16", L=8, n=2, Ls=2, Hq=4, Hkv=2, hd=128, F=512, V=700, anchors=[0, 4, 8],
                           attn_period=4, p=0.7, seed=73),
    "f32_n1": dict(L=4, n=1, Ls=2, anchors=[0, 2, 4], attn_period=4, G=16, p=0.6, seed=74),
}


@pytest.mark.parametrize("name", sorted(HYBRID))
def test_hybrid_matches_oracle(name):
    kw = dict(HYBRID[name])
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
    acc = recs["accepted"][recs["exit_pos"] >= 0]
    assert (acc == 1).any() and (acc == 0).any()


def test_hybrid_sampling_matches_oracle():
    w = gpu_workload_tiny(mode="sample", temperature=1.0, L=4, n=2, anchors=[0, 2, 3], attn_period=2, seed=75)
    T, W, prompt, uni = _inputs(w)
    eng, first, recs, toks = run_gpu(w, T, prompt, uni=uni)
    eng.close()
    o = SPDOracle(w, W, uniforms=uni, teacher=teacher_of(recs, first), tol=TOL[w.dtype], sample_tol=STOL[w.dtype])
    otoks, ologs = o.run(prompt, w.G)
    assert not o.dec.mismatch, o.dec.mismatch
    assert len(o.dec.adopted) <= 2
    assert toks == otoks
    compare_logs(recs, ologs, w.L)


def test_hybrid_lossless_through_the_prefill_checkpoint():
    """Forced and natural drafts equal the GPU's autoregressive decode, which
    ran past the state ring first (the rollback restores the prefill states)."""
    w = gpu_workload_tiny(dtype="bf16", L=8, n=4, Ls=2, anchors=[0, 2, 4, 6, 8], attn_period=4, G=30, seed=76)
    T, W, prompt, uni = _inputs(w)
    from pipelined_draft_verify_amd import SPDEngine, SPDError

    eng = SPDEngine(w, {k: v.to("cuda:0") for k, v in T.items()})
    eng.set_uniforms(uni)
    first = eng.prefill(prompt)
    ar = eng.generate_ar(w.G - 1)
    ref = list(prompt) + [first] + ar
    # a length between the prefill and the ring's reach is gone
    with pytest.raises(SPDError):
        eng.rollback(w.P + 3, ar[2])
    for p in (None, 0.0, 0.5, 1.0):
        eng.rollback(w.P, first)
        if p is not None:
            eng.set_forced(ref, p)
        recs = eng.run()
        assert eng.tokens(w.P, w.G) == [first] + ar, p
        if p == 1.0:
            assert (recs["accepted"][recs["exit_pos"] >= 0] == 1).all()
    eng.close()
