"""Pins of the draft-tree oracle (oracle/tree.py; CPU only).

[RB] prerequisites ("draft tree": keep the top-W branches by cumulative
probability) and [PL] appendix B (each SPD draft step widened into a width-4
tree); the tree's verification and per-branch KV follow the reading in the
module header.  Pinned by:

  * W = 1 is the single-draft pipeline of oracle.spd, integer for integer and
    bit for bit in the verification and draft logits (and the KV lengths,
    once the tree's committed length is counted with the in-flight tokens);
  * losslessness by brute force: for widths 2-4, random tiny models and
    forced tree policies of every kind, the output equals the target's greedy
    autoregressive decoding and the committed KV equals the AR KV;
  * the cycle count obeys the same closed form as the chain;
  * each node's state equals a plain forward of its own path: the exiting
    node's logits equal the AR target logits, and the draft module's row of
    every leaf equals the chain computation over that leaf's path alone;
  * the entered nodes are the top-W pairs (surviving leaf, token) by the
    product of draft probabilities along the path, by brute force over every
    surviving leaf and every token with torch's float64 softmax;
  * the tree's shape: at most W nodes per position, one at the oldest, every
    node a child of the previous position, the accepted child kept;
  * planted mistakes (no pruning, all-rows draft attention, a sibling's KV,
    a ranking without the path probability) are caught.
"""
import numpy as np
import pytest

import seeded_inputs as si
from oracle import ForcedPolicy, SPDOracle, ar_greedy, schedule
from oracle import tree as TR
from oracle.model import layer_rows
from oracle.tree import TreeForcedPolicy, TreeSPDOracle

MODELS = [
    dict(L=4, n=2, Ls=1, anchors=[0, 2, 3], Hq=4, Hkv=2, seed=11),
    dict(L=4, n=4, Ls=1, anchors=[0, 1, 2, 4], Hq=2, Hkv=2, seed=12),
    dict(L=6, n=3, Ls=2, anchors=[0, 1, 4, 6], Hq=4, Hkv=1, seed=13),
    dict(L=8, n=4, Ls=2, anchors=[0, 2, 4, 6, 7], Hq=4, Hkv=4, seed=14, dtype="bf16"),
    dict(L=8, n=8, Ls=1, anchors=[0, 3, 8], Hq=6, Hkv=3, seed=15, norm_gain="random"),
]
POLICIES = {"wrong": (0.0, 0.0), "tree_only": (0.0, 0.7), "mixed": (0.3, 0.8), "right": (1.0, 1.0),
            "chain": (0.5, 0.5)}


def _setup(G=16, **kw):
    w = si.tiny(G=G, **kw)
    W = si.nest_weights(si.weights_numpy_f32(si.make_weights(w)), w)
    prompt = si.make_prompt(w)
    u = si.make_uniforms(w)
    ref, tgt = ar_greedy(w, W, prompt, w.G)
    return w, W, prompt, u, ref, tgt


@pytest.mark.parametrize("mi", range(len(MODELS)))
@pytest.mark.parametrize("p", [None, 0.0, 0.4, 1.0])
def test_width_one_is_the_single_draft_pipeline(mi, p):
    w, W, prompt, u, ref, _ = _setup(**MODELS[mi])
    lin = SPDOracle(w, W, policy=None if p is None else ForcedPolicy(ref, p, u, w.V), uniforms=u)
    tre = TreeSPDOracle(w, W, 1, policy=None if p is None else TreeForcedPolicy(ref, p, p, u, w.V))
    fl, ft = {}, {}
    lin.hook = lambda k, i: fl.setdefault((k, i["cycle"]), i["logits"].copy())
    tre.hook = lambda k, i: ft.setdefault((k, i["cycle"]), i["logits"].copy()) if k in ("exit", "pdm") else None
    lt, ll = lin.run(prompt, w.G)
    tt, tl = tre.run(prompt, w.G)
    assert lt == tt
    assert len(ll) == len(tl)
    for a, b in zip(ll, tl):
        assert (a["t"], a["a"], a["pending_row"], a["exit_pos"], a["y"], a["accept"], a["pdm_len"], a["emitted"]) == \
            (b["t"], b["a"], b["pending_row"], b["exit_pos"], b["y"], b["accept"], b["pdm_len"], b["emitted"])
        assert b["nodes"] == a["a"]
        # the chain's per-layer length: committed + in-flight tokens that passed the layer
        inflight = list(range(b["t"] - b["a"] + 1, b["t"] + 1))
        if b["exit_pos"] >= 0 and b["accept"] == 1:
            inflight = inflight[1:]
        if b["exit_pos"] >= 0 and b["accept"] == 0:
            inflight = []
        for l in range(w.L):
            passed = sum(1 for q in inflight if schedule.stage_layers(b["t"] - q, w.L, w.n).stop > l)
            assert a["kv_len"][l] == b["committed"] + passed, (a["cycle"], l)
    for c in range(len(tl)):
        if tl[c]["exit_pos"] >= 0 or ll[c]["accept"] >= 0:
            pass
    # verification and draft logits, bit for bit
    for key, v in fl.items():
        assert np.array_equal(v, ft[key]), key
    # the draft: the chain's draft is the tree's single entered node of the next cycle
    for a, b in zip(ll[:-1], tl[1:]):
        if a["exit_pos"] < 0 or a["accept"] == 1:
            assert b["new_token"] == [a["draft"]]


def _runs(mi, Wd):
    w, W, prompt, u, ref, tgt = _setup(**MODELS[mi])
    for name, (p1, pW) in POLICIES.items():
        o = TreeSPDOracle(w, W, Wd, policy=TreeForcedPolicy(ref, p1, pW, u, w.V))
        yield name, w, ref, tgt, o, o.run(prompt, w.G)
    o = TreeSPDOracle(w, W, Wd)
    yield "natural", w, ref, tgt, o, o.run(prompt, w.G)


@pytest.mark.parametrize("mi", range(len(MODELS)))
@pytest.mark.parametrize("Wd", [2, 3, 4])
def test_lossless_and_cycle_count(mi, Wd):
    for name, w, ref, tgt, o, (toks, logs) in _runs(mi, Wd):
        assert toks == ref, name
        # the committed KV is the autoregressive KV of the verified prefix
        m = o.committed()
        for l in range(w.L):
            assert np.array_equal(o.target.kv[l].K[:m], tgt.kv[l].K[:m]), (name, l)
            assert np.array_equal(o.target.kv[l].V[:m], tgt.kv[l].V[:m]), (name, l)
        ver = [x for x in logs if x["exit_pos"] >= 0]
        R = sum(1 for x in ver[: w.G - 2] if not x["accept"])
        assert len(logs) == schedule.cycle_count(w.n, w.G, R), name
        assert [x["exit_pos"] for x in ver] == list(range(w.P, w.P + w.G - 1))


@pytest.mark.parametrize("mi", [1, 2, 4])
def test_tree_shape(mi):
    w, W, prompt, u, ref, _ = _setup(**MODELS[mi])
    Wd = 3
    o = TreeSPDOracle(w, W, Wd, policy=TreeForcedPolicy(ref, 0.2, 0.7, u, w.V))
    o.prefill(prompt)
    widths = []
    while o.emitted < w.G:
        rec = o.cycle()
        pos = sorted(o.levels)
        if not pos:
            continue
        assert len(o.levels[pos[0]]) == 1
        for p in pos:
            assert 1 <= len(o.levels[p]) <= Wd
            for nd in o.levels[p]:
                assert nd.pos == p
                if p > pos[0]:
                    assert any(nd.parent is x for x in o.levels[p - 1])
        widths.append(max(len(o.levels[p]) for p in pos))
        if rec["accept"] == 1:
            kept = o.levels[rec["exit_pos"] + 1][0]
            assert kept.tok == rec["y"]
    assert max(widths) == Wd  # the tree does widen


@pytest.mark.parametrize("mi", [2, 3, 4])
def test_node_states_follow_their_own_paths(mi):
    """The exiting node's logits are the autoregressive logits of its
    position, and the draft module's row of every leaf equals the chain
    computation over the committed prefix and that leaf's path alone."""
    w, W, prompt, u, ref, _ = _setup(**MODELS[mi])
    o = TreeSPDOracle(w, W, 3, policy=TreeForcedPolicy(ref, 0.3, 0.8, u, w.V))
    from oracle.model import Target
    ar = Target(w, W)
    ar_logits = {}
    for p_, tok in enumerate(ref[:-1]):
        h, _ = ar.forward_token(int(tok), p_)
        ar_logits[p_] = ar.logits(h)
    seen = {"exit": 0, "leaf": 0}

    def hook(kind, info):
        if kind == "exit":
            assert np.array_equal(info["logits"], ar_logits[info["pos"]])
            seen["exit"] += 1
        elif kind == "pdm_rows":
            rows, G, X, C = info["rows"], info["G"], info["X"], info["C"]
            t = max(nd.pos for nd, _ in rows)
            for li, (nd, _) in enumerate(rows):
                if nd.pos != t:
                    continue
                chain = [r for r, (x, _) in enumerate(rows) if x is nd or (x.pos < nd.pos and x in _ancestors(nd))]
                chain = sorted(chain, key=lambda r: rows[r][0].pos)
                assert [rows[r][0].pos for r in chain] == list(range(C, t + 1))
                Y = _chain_pdm(o, G[chain], C)
                assert np.array_equal(Y[-1], X[li])
                seen["leaf"] += 1

    o.hook = hook
    o.run(prompt, w.G)
    assert seen["exit"] >= 5 and seen["leaf"] >= 10


def _ancestors(nd):
    out, x = [], nd.parent
    while x is not None:
        out.append(x)
        x = x.parent
    return out


def _chain_pdm(o, G, C):
    """The draft module's layers over one chain of rows at positions C.. with
    the committed prefix (oracle.model.layer_rows on a scratch copy of the KV)."""
    import copy
    kvs = [copy.deepcopy(kv) for kv in o.pdm.kv]
    X = G.astype(np.float32)
    for l in range(o.s.Ls):
        X = layer_rows(o.s, o.pdm.W["pdm_layers"][l], X, C, kvs[l])
    return X


def test_tree_catches_second_ranked_drafts():
    """With p1 = 0 the true token is never ranked first; a chain would reject
    every verification, the tree (W >= 2) accepts at rate ~pW."""
    w, W, prompt, u, ref, _ = _setup(G=40, **MODELS[1])
    for Wd, want in ((1, 0.0), (3, 0.8)):
        o = TreeSPDOracle(w, W, Wd, policy=TreeForcedPolicy(ref, 0.0, 0.8, u, w.V))
        toks, logs = o.run(prompt, w.G)
        assert toks == ref
        acc = np.mean([x["accept"] for x in logs if x["exit_pos"] >= 0])
        if Wd == 1:
            assert acc < 0.2
        else:
            assert acc > 0.5


# -- planted mistakes --------------------------------------------------------
def test_no_pruning_is_caught(monkeypatch):
    """Keeping every child after an accepted verification leaves several
    nodes at the oldest position: the run's invariants catch it."""
    w, W, prompt, u, ref, _ = _setup(**MODELS[1])
    monkeypatch.setattr(TreeSPDOracle, "_prune_to", lambda self, keep, j: None)
    o = TreeSPDOracle(w, W, 3, policy=TreeForcedPolicy(ref, 0.2, 0.9, u, w.V))
    with pytest.raises(AssertionError):
        o.run(prompt, w.G)


def test_draft_attention_over_all_rows_is_caught(monkeypatch):
    """Attending to every trailing row up to the position (not only the
    ancestors) breaks the per-path equality of the draft module's rows."""
    def bad(self, G, rows):
        # chain-style attention over the rows in row order
        s, pdm = self.s, self.pdm
        C = pdm.C
        import copy
        kvs = [copy.deepcopy(kv) for kv in pdm.kv]
        X = G.astype(np.float32)
        for l in range(s.Ls):
            kvs[l].K[C:C + len(rows)] = 0
            X = layer_rows(s, pdm.W["pdm_layers"][l], X, C, kvs[l])
        return X

    monkeypatch.setattr(TreeSPDOracle, "_pdm_layers", bad)
    with pytest.raises(AssertionError):
        test_node_states_follow_their_own_paths(2)


def test_sibling_kv_is_caught(monkeypatch):
    """A node that attends to a sibling branch's key/values (the first node
    at each ancestor position) no longer follows its own path."""
    orig_path = TR.Node.path

    def wrong_path(self, stop):
        out = orig_path(self, stop)
        return out
    orig_run = TreeSPDOracle._run_stage

    def bad_run(self, nd, k, F):
        if nd.parent is not None and nd.parent.pos in self.levels and len(self.levels[nd.parent.pos]) > 1:
            sib = self.levels[nd.parent.pos][0] if self.levels[nd.parent.pos][0] is not nd.parent \
                else self.levels[nd.parent.pos][1]
            saved = nd.parent
            nd.parent = sib
            try:
                orig_run(self, nd, k, F)
            finally:
                nd.parent = saved
            return
        orig_run(self, nd, k, F)

    monkeypatch.setattr(TreeSPDOracle, "_run_stage", bad_run)
    with pytest.raises(AssertionError):
        test_node_states_follow_their_own_paths(2)


# -- the ranking: top-W branches by cumulative probability -------------------
def test_log_softmax64_matches_torch():
    import torch
    rng = np.random.default_rng(5)
    for V in (7, 300, 4096):
        l = (rng.standard_normal(V) * rng.uniform(0.1, 30)).astype(np.float32)
        want = torch.log_softmax(torch.from_numpy(l.astype(np.float64)), 0).numpy()
        assert np.allclose(TR.log_softmax64(l), want, rtol=0, atol=1e-12)


def _entries_by_brute_force(mi, Wd, G=24):
    """Run the tree with its own draft module (no forcing) and, at every
    cycle that enters drafted nodes, compare the entered (parent, token)
    pairs with the top-W pairs over ALL surviving leaves and ALL tokens by
    the product of draft probabilities along the path, the probabilities
    taken by torch's float64 softmax of the logits each parent leaf had
    when it drafted.  Returns the number of cycles checked."""
    import torch
    w, W, prompt, u, ref, _ = _setup(G=G, **MODELS[mi])
    o = TreeSPDOracle(w, W, Wd)
    logits = {}  # id(leaf) -> draft logits of the cycle it was a leaf in

    def hook(kind, info):
        if kind == "pdm":
            logits[id(info["leaf"])] = info["logits"]

    o.hook = hook
    o.prefill(prompt)

    def prob(x):
        if id(x.parent) not in logits:     # a re-seeded or verified root: common to every path
            return 1.0
        p = torch.softmax(torch.from_numpy(logits[id(x.parent)].astype(np.float64)), 0)
        return float(p[x.tok])

    checked = 0
    while o.emitted < w.G:
        # the leaves that survived the last verification: the next entry drafts from them
        leaves = list(o.levels[max(o.levels)]) if o.levels and o.reseed is None else []
        rec = o.cycle()
        if not leaves:
            continue
        assert rec["new_parent"][0] >= 0
        pool = []
        for lf in leaves:
            path_p = 1.0
            x = lf
            while x is not None:
                path_p *= prob(x)
                x = x.parent
            q = torch.softmax(torch.from_numpy(logits[id(lf)].astype(np.float64)), 0).numpy()
            for tok in range(w.V):
                pool.append((path_p * q[tok], lf, tok))
        pool.sort(key=lambda e: -e[0])
        want = {(id(lf), tok) for _, lf, tok in pool[:Wd]}
        got = {(id(leaves[pr]), tok) for pr, tok in zip(rec["new_parent"], rec["new_token"])}
        assert got == want, (rec["cycle"], got, want)
        checked += 1
    return checked


@pytest.mark.parametrize("mi,Wd", [(0, 2), (1, 4), (3, 3)])
def test_entries_are_the_top_branches_by_cumulative_probability(mi, Wd):
    assert _entries_by_brute_force(mi, Wd) >= 5


def test_ranking_without_the_path_probability_is_caught(monkeypatch):
    """Ranking every leaf's candidates by their own draft probability alone
    (dropping the path's cumulative probability) picks other branches."""
    orig = TR.Node.path

    def short_path(self, stop):
        out = orig(self, stop)
        import inspect
        if inspect.stack()[1].function == "_draft":
            return out[-1:]            # cum = the leaf's own log probability only
        return out

    monkeypatch.setattr(TR.Node, "path", short_path)
    with pytest.raises(AssertionError):
        for mi, Wd in [(0, 2), (1, 4), (3, 3)]:
            _entries_by_brute_force(mi, Wd)
