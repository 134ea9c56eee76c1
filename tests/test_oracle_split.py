"""Pins of the non-uniform stage split (CPU only).

Per-stage layer counts, as in the pages' "5+4;9;9;9" example (a 5-layer
first stage sharing its rank with the 4-layer draft module, then three
9-layer stages): the closed forms of lmax, f(k) and the stage ranges; a
uniform split written out reproduces the uniform schedule; and, by brute
force over draft policies, SPD with uneven stages still emits exactly the
target's greedy decode, with every stage's KV lengths and the cycle count of
the uniform case, and the integer replay reproduces every cycle.
"""
import numpy as np
import pytest

from oracle import SPDOracle, ar_greedy
from oracle import schedule as S
from oracle.model import PDM
from tests.test_oracle_replay import _replay, _same
from tests.test_oracle_spd import _policies, _rejects_before_last, _setup

ANCHORS = [0, 8, 16, 24, 31]


def test_the_5_9_9_9_split():
    split = [5, 9, 9, 9]
    assert S.stage_sizes(32, 4, split) == split
    assert [S.lmax(k, 32, 4, split) for k in range(5)] == [0, 5, 14, 23, 32]
    # depth 1 (5 layers) reaches no anchor past the embedding; the anchor at
    # 24 is reached by no depth (23 < 24 < 32), so only 4 projections are used
    assert S.pattern_table(ANCHORS, 32, 4, split) == [0, 0, 1, 2, 4]
    assert S.n_patterns(ANCHORS, 32, 4, split) == 4
    assert [S.stage_layers(k, 32, 4, split) for k in range(4)] == [range(0, 5), range(5, 14), range(14, 23),
                                                                   range(23, 32)]
    S.validate_shape(32, 4, 4, ANCHORS, split)  # the example's 4-layer draft module
    S.validate_shape(32, 4, 9, ANCHORS, split)  # as deep as the longest stage
    for Ls, bad in [(10, split), (4, [5, 9, 9, 8]), (4, [0, 14, 9, 9]), (4, [5, 9, 18])]:
        with pytest.raises(ValueError):
            S.validate_shape(32, 4, Ls, ANCHORS, bad)


@pytest.mark.parametrize("L,n", [(32, 8), (32, 16), (32, 4), (8, 4), (6, 3), (12, 1)])
def test_a_uniform_split_written_out_is_the_uniform_schedule(L, n):
    anchors = [0, L // 3, L // 2, L - 1] if L > 6 else [0, 1, 4, 6]
    split = [L // n] * n
    assert S.pattern_table(anchors, L, n, split) == S.pattern_table(anchors, L, n)
    assert [S.lmax(k, L, n, split) for k in range(n + 1)] == [S.lmax(k, L, n) for k in range(n + 1)]
    assert [S.stage_layers(k, L, n, split) for k in range(n)] == [S.stage_layers(k, L, n) for k in range(n)]


SPLITS = [
    dict(L=6, n=3, split=(1, 3, 2), Ls=2, anchors=[0, 1, 4, 6], Hq=4, Hkv=1, seed=21),
    dict(L=8, n=4, split=(3, 1, 2, 2), Ls=3, anchors=[0, 2, 4, 6, 7], Hq=4, Hkv=2, seed=22, dtype="bf16"),
    dict(L=5, n=2, split=(4, 1), Ls=1, anchors=[0, 3, 5], Hq=2, Hkv=2, seed=23),
    dict(L=6, n=3, split=(2, 1, 3), Ls=3, anchors=[0, 1, 4, 6], Hq=4, Hkv=2, seed=24),
]


@pytest.mark.parametrize("mi", range(len(SPLITS)))
def test_uneven_stages_are_lossless(mi):
    w, W, prompt, u = _setup(G=14, **SPLITS[mi])
    S.validate_shape(w.L, w.n, w.Ls, w.anchors, w.split)
    ref, ar = ar_greedy(w, W, prompt, w.G)
    stage_of = [k for k in range(w.n) for _ in S.stage_layers(k, w.L, w.n, w.split)]
    for name, pol in _policies(w, ref, u).items():
        o = SPDOracle(w, W, policy=pol, uniforms=u)
        toks, logs = o.run(prompt, w.G)
        assert toks == ref, name
        upto = len(ref) - 1
        for l in range(w.L):
            m = min(upto, o.target.kv[l].length)
            assert np.array_equal(o.target.kv[l].K[:m], ar.kv[l].K[:m]), (name, l)
            assert np.array_equal(o.target.kv[l].V[:m], ar.kv[l].V[:m]), (name, l)
        assert len(logs) == S.cycle_count(w.n, w.G, _rejects_before_last(logs, w.G)), name
        for lg in logs:
            t, a = lg["t"], lg["a"]
            if lg["exit_pos"] >= 0 and not lg["accept"]:
                assert lg["kv_len"] == [lg["exit_pos"] + 1] * w.L
            else:
                assert lg["kv_len"] == [t + 1 - min(stage_of[l], a) for l in range(w.L)], (name, lg)
        _same(logs, _replay(w, toks[w.P], logs, pol))


def test_split_changes_the_features():
    """The split is not ignored: the draft module's feature of a depth whose
    lmax moves past an anchor uses another fusion pattern."""
    w0, W, _, _ = _setup(L=6, n=3, Ls=2, anchors=[0, 1, 4, 6], Hq=4, Hkv=1, seed=21)
    w1 = w0.replace(split=(2, 1, 3))
    assert S.pattern_table(w0.anchors, 6, 3) == [0, 1, 2, 3]
    assert S.pattern_table(w1.anchors, 6, 3, w1.split) == [0, 1, 1, 3]
    rng = np.random.default_rng(0)
    taps = [rng.standard_normal(w0.d).astype(np.float32) for _ in w0.anchors]
    p0, p1 = PDM(w0, W), PDM(w1, W)
    for k in range(4):
        assert np.array_equal(p0.feature(taps, k), p1.feature(taps, k)) == (k != 2), k
