"""GPU parity over seeded random small configurations.

Each case draws a valid shape and mode from a fixed seed -- dtype, stage count,
uniform or uneven stage split, draft-module depth, anchor set, head layout,
vocabulary, greedy with forced drafts or temperature sampling (optionally
top-k), pre- or post-step drafting, hybrid linear-attention layers -- and must
agree with the oracle cycle by cycle as in the hand-picked small variants.
Sixteen more cases draw draft-tree configurations (width 2-4, up to eight
stages, forced tree policies or the draft module's own drafts) and follow
the tree oracle cycle by cycle.  The point is the combinations no single
variant covers.  Three medium cases
(widths 1024-2048, prompts of 260-620 tokens, vocabularies up to 32000) add
several tiles per stage group and multi-split attention.
"""
import numpy as np
import pytest

from oracle import SPDOracle, ar_greedy
from tests.gpu_common import compare_logs, gpu_workload_tiny, run_gpu, teacher_of
from tests.test_gpu_parity_small import STOL, TOL, _inputs, _oracle

pytestmark = pytest.mark.gpu

N_CASES = 48


def _draw(i):
    rng = np.random.default_rng(2026 + i)
    n = int(rng.choice([1, 2, 3, 4, 6]))
    if rng.random() < 0.5:
        L = n * int(rng.integers(1, 4))
        split = ()
    else:
        L = int(rng.integers(n, n + 7))
        cuts = sorted(rng.choice(np.arange(1, L), size=n - 1, replace=False)) if n > 1 else []
        edges = [0] + [int(c) for c in cuts] + [L]
        split = tuple(edges[k + 1] - edges[k] for k in range(n))
    longest = max(split) if split else L // n
    Ls = int(rng.integers(1, min(longest, 8) + 1))
    inner = sorted(set(int(b) for b in rng.integers(1, L + 1, size=int(rng.integers(0, 5)))))
    anchors = [0] + inner[:7]
    Hq, Hkv, hd = [(4, 2, 64), (4, 4, 64), (8, 2, 64), (2, 1, 128), (4, 1, 128)][int(rng.integers(0, 5))]
    kw = dict(dtype=str(rng.choice(["f32", "bf16"])), L=L, n=n, Ls=Ls, anchors=anchors, Hq=Hq, Hkv=Hkv, hd=hd,
              d=int(rng.choice([256, 512])), F=int(rng.choice([512, 768])), V=int(rng.choice([300, 997, 2048])),
              P=int(rng.integers(5, 41)), G=int(rng.integers(8, 25)), seed=100 + i, split=split)
    if n >= 2 and rng.random() < 0.25:
        kw["schedule"] = "post"
    if rng.random() < 0.3:
        period = int(rng.choice([2, 4]))
        if period <= L:  # the library takes attn_period <= n_layers
            kw["attn_period"] = period
    if rng.random() < 0.35:
        kw.update(mode="sample", temperature=float(rng.choice([0.5, 1.0])), top_k=int(rng.choice([0, 0, 8])))
        p = None
    else:
        p = float(rng.choice([0.3, 0.7]))
    return kw, p


def _draw_medium(i):
    """Larger shapes: several tiles per stage group, prompts long enough for
    two or three attention splits, vocabularies of several sampler superblocks."""
    rng = np.random.default_rng(5000 + i)
    n = int(rng.choice([2, 4, 8]))
    L = 8 if n < 8 else 8 * int(rng.integers(1, 3))
    split = ()
    if n < 8 and rng.random() < 0.5:
        cuts = sorted(rng.choice(np.arange(1, L), size=n - 1, replace=False))
        edges = [0] + [int(c) for c in cuts] + [L]
        split = tuple(edges[k + 1] - edges[k] for k in range(n))
    longest = max(split) if split else L // n
    Hq, Hkv, hd = [(16, 4, 128), (8, 8, 128), (32, 8, 64)][int(rng.integers(0, 3))]
    kw = dict(dtype="bf16", L=L, n=n, Ls=int(rng.integers(1, longest + 1)),
              anchors=[0] + sorted(set(int(b) for b in rng.integers(1, L + 1, size=3))),
              Hq=Hq, Hkv=Hkv, hd=hd, d=int(rng.choice([1024, 2048])), F=int(rng.choice([2048, 4096])),
              V=int(rng.choice([4096, 32000])), P=int(rng.integers(260, 620)), G=int(rng.integers(10, 17)),
              seed=300 + i, split=split)
    if rng.random() < 0.4:
        kw.update(mode="sample", temperature=1.0, top_k=int(rng.choice([0, 50])))
        p = None
    else:
        p = float(rng.choice([0.5, 0.8]))
    return kw, p


CASES = [("small", i) for i in range(N_CASES)] + [("medium", i) for i in range(3)]


@pytest.mark.parametrize("kind,i", CASES)
def test_random_configuration_matches_oracle(kind, i):
    kw, p = (_draw if kind == "small" else _draw_medium)(i)
    print("case", kind, i, kw, "p", p, flush=True)
    w = gpu_workload_tiny(**kw)
    T, W, prompt, uni = _inputs(w)
    if w.mode == "sample":
        eng, first, recs, toks = run_gpu(w, T, prompt, uni=uni)
        eng.close()
        o = SPDOracle(w, W, uniforms=uni, teacher=teacher_of(recs, first), tol=TOL[w.dtype],
                      sample_tol=STOL[w.dtype])
        otoks, ologs = o.run(prompt, w.G)
    else:
        ref, _ = ar_greedy(w, W, prompt, w.G)
        eng, first, recs, toks = run_gpu(w, T, prompt, uni=uni, ref=ref, p_accept=p)
        eng.close()
        # forced drafts follow the oracle's own greedy decode; the GPU's tokens
        # are its own greedy decode, equal to it up to near-ties (checked below)
        o, otoks, ologs = _oracle(w, W, prompt, uni, recs, first, ref=ref, p=p)
    assert not o.dec.mismatch, o.dec.mismatch
    assert len(o.dec.adopted) <= 2, o.dec.adopted
    assert toks == otoks
    compare_logs(recs, ologs, w.L)


# ---- draft trees ----------------------------------------------------------
N_TREE_CASES = 16


def _draw_tree(i):
    """A random draft-tree configuration (greedy, pre-step, uniform stages,
    2 + (n - 1) W <= 32 draft-module rows), with a forced tree policy or the
    draft module's own drafts."""
    rng = np.random.default_rng(7000 + i)
    while True:
        n = int(rng.choice([2, 3, 4, 6, 8]))
        Wd = int(rng.choice([2, 3, 4]))
        if 2 + (n - 1) * Wd <= 32:
            break
    L = n * int(rng.integers(1, 3))
    Ls = int(rng.integers(1, L // n + 1))
    inner = sorted(set(int(b) for b in rng.integers(1, L + 1, size=int(rng.integers(0, 4)))))
    Hq, Hkv, hd = [(4, 2, 64), (4, 4, 64), (8, 2, 64), (2, 1, 128), (4, 1, 128)][int(rng.integers(0, 5))]
    kw = dict(dtype=str(rng.choice(["f32", "bf16"])), L=L, n=n, Ls=Ls, anchors=[0] + inner[:7], Hq=Hq, Hkv=Hkv,
              hd=hd, d=int(rng.choice([256, 512])), F=int(rng.choice([512, 768])),
              V=int(rng.choice([300, 997, 2048])), P=int(rng.integers(5, 41)), G=int(rng.integers(10, 25)),
              seed=700 + i, width=Wd)
    if rng.random() < 0.25:
        return kw, None, None
    return kw, float(rng.choice([0.0, 0.3, 0.5])), float(rng.choice([0.6, 0.85]))


@pytest.mark.parametrize("i", range(N_TREE_CASES))
def test_random_tree_configuration_matches_oracle(i):
    from tests.test_gpu_tree import run_and_compare

    kw, p1, pW = _draw_tree(i)
    print("tree case", i, kw, "p1", p1, "pW", pW, flush=True)
    w = gpu_workload_tiny(**kw)
    T, W, prompt, uni = _inputs(w)
    ref, _ = ar_greedy(w, W, prompt, w.G)
    recs, ologs, o = run_and_compare(w, T, W, prompt, uni, ref, p1, pW)
    assert len(o.adopted) <= 3, o.adopted
    assert recs["n_new"].max() >= 2  # the tree widens
