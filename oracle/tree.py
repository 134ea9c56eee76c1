"""Draft trees inside the SPD pipeline (test infrastructure only).

[RB] prerequisites ("draft tree"): the draft module proposes several branch
candidates at once, forming a tree that widens what one verification covers;
the usual rule keeps the top-W branches by cumulative probability, each node
expanding into children.  [PL] appendix B widens each draft step of SPD into
a width-4 tree; [PL] §4 and [RB] limitations leave the wall-clock system --
branch scheduling, per-branch KV caches, cross-stage synchronisation -- open.

Reading taken here (greedy verification, pre-step drafting, n >= 2):

  * the tokens in flight form a tree rooted at the oldest in-flight token,
    which is always a single verified token; every in-flight position holds
    at most W nodes, all children of nodes at the previous position;
  * every cycle the draft module runs on the pre-step features of every
    in-flight node (the just-verified row at depth n, each node at depth
    t - position), each row attending to the committed draft-module prefix,
    to its own ancestors and to itself; the leaves (the nodes at the newest
    position t) each give a draft distribution Q_leaf = softmax(logits);
  * candidates for position t+1 are the pairs (leaf, token) with the leaf's
    W most likely tokens; a pair scores cum(leaf) + log Q_leaf(token), where
    cum sums log Q over the leaf's in-flight path (a constant shared by all
    leaves is left out); candidates are ranked by score (ties: lower leaf
    rank, then lower token id);
  * drafting runs beside the stage step and verification prunes branches in
    the same cycle, so the next cycle enters the first W candidates whose leaf
    survived, in rank order; they enter stage 0 together, and every in-flight
    node that is no longer on a path to one of them (a branch that got no
    child) is dropped;
  * the stage step advances every node through its own stage; a node attends
    to the committed prefix, its ancestors and itself (per-branch KV);
  * the single node at the oldest position exits and verifies its children:
    the child whose token is the target's argmax is kept (every other
    subtree is pruned); if no child matches, the three-step rollback runs
    (truncate every layer's KV to j+1, flush the tree, re-seed stage 0);
  * the exiting node's KV joins the committed cache; the committed length is
    the same in every layer (the tree's KV is per node until it exits).

With W = 1 the tree is the single in-flight chain and the run is the
pipeline of oracle.spd step for step (a pin in the CPU tests).

Forced acceptance for trees (harness device, not on the pages): with the
target's greedy continuation R and the forced leaf (the leaf whose path,
from the oldest in-flight position, matches R for the longest prefix; ties
to the lower rank), the draw
u = U[q, FORCE] for position q places the pair (forced leaf, R[q]) first in
the ranking when u < p1, at rank W-1 when p1 <= u < pW and W >= 2 (only a
tree catches it), and otherwise removes it (its token is replaced by the
next id not already a candidate of that leaf) while keeping the forced
leaf's branch alive: if none of its candidates is among the first W, such a
wrong child is put at rank W-1 (a draft module that keeps the true branch
but misses its next token, as one draft per cycle does).  With W = 1 this is
the single-draft forced policy with p = p1.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import numpy as np

from seeded_inputs import U_FORCE

from .layers import F32, apply_rope, attention, rope_cos_sin
from .model import PDM, Target, _ffn, _qkv
from .layers import rmsnorm
from .schedule import depth_layout, stage_layers


class Node:
    """One in-flight token of the tree."""

    def __init__(self, pos: int, tok: int, parent: Optional["Node"], logq: float):
        self.pos, self.tok, self.parent, self.logq = pos, tok, parent, logq
        self.h = None
        self.taps: list = []
        self.kv: Dict[int, tuple] = {}  # target layer -> (k, v) of this node

    def path(self, stop: int) -> List["Node"]:
        """Ancestors at positions > stop, oldest first, then the node itself."""
        out, x = [], self
        while x is not None and x.pos > stop:
            out.append(x)
            x = x.parent
        return out[::-1]


def log_softmax64(logits: np.ndarray) -> np.ndarray:
    """log softmax in float64 (the draft probabilities the ranking uses)."""
    l = logits.astype(np.float64)
    m = l.max()
    return l - m - np.log(np.sum(np.exp(l - m)))


class TreeForcedPolicy:
    def __init__(self, ref: Sequence[int], p1: float, pW: float, uniforms: np.ndarray, V: int):
        self.ref = [int(x) for x in ref]
        self.p1, self.pW = np.float32(p1), np.float32(pW)
        self.u = uniforms
        self.V = V


def _step_layer(s, lw, h, pos, Kp, Vp, bf16):
    """One target layer for one node: keys/values of positions < pos are
    given (committed prefix then ancestors); returns (h, k, v)."""
    u = rmsnorm(h, lw["attn_norm"], s.eps)
    q, k, v = _qkv(lw, u, s.Hq, s.Hkv, s.hd)
    c, sn = rope_cos_sin(pos, s.hd, s.base)
    q, k = apply_rope(q, c, sn), apply_rope(k, c, sn)
    if bf16:
        from .layers import bf16_round
        k, v = bf16_round(k), bf16_round(v)
    K = np.concatenate([Kp, k[None]], axis=0)
    V = np.concatenate([Vp, v[None]], axis=0)
    o = attention(q, K, V)
    h = h + lw["w_o"] @ o.reshape(-1)
    return _ffn(lw, h, s.F, s.eps), k, v


class TreeSPDOracle:
    """SPD with a width-W draft tree (greedy), one cycle at a time."""

    def __init__(self, w, W, width: int, policy: Optional[TreeForcedPolicy] = None,
                 teacher: Optional[Dict] = None, tol: float = 0.0):
        if w.mode != "greedy" or getattr(w, "schedule", "pre") != "pre":
            raise ValueError("draft trees: greedy verification, pre-step drafting")
        if w.n < 2:
            raise ValueError("draft trees need n >= 2")
        if getattr(w, "attn_period", 0):
            raise ValueError("draft trees: softmax-attention targets only")
        self.w, self.Wd = w, width
        self.n, self.L, self.V = w.n, w.L, w.V
        self.target = Target(w, W)
        self.pdm = PDM(w, W)
        self.s = self.target.s
        self.policy = policy
        self.teacher = teacher
        self.tol = tol
        self.adopted: List[tuple] = []
        self.mismatch: List[tuple] = []
        self.levels: Dict[int, List[Node]] = {}  # in-flight position -> nodes in rank order
        self.cands: List[tuple] = []             # (leaf, token, score) ranked, from the last draft step
        self.pending: Optional[Node] = None      # exited node whose draft-module row is committed next
        self.reseed = None
        self.tokens: List[int] = []
        self.emitted = 0
        self.ncycles = 0
        self.logs: List[dict] = []
        self.P = 0
        self.hook = None

    # -- prefill (as oracle.spd: full target pass, first token, draft-module prefill)
    def prefill(self, prompt: Sequence[int], matrix: bool = False) -> int:
        self.P = len(prompt)
        if matrix:
            h, full = self.target.prefill_matrix([int(t) for t in prompt])
        else:
            full = []
            for p, tok in enumerate(prompt):
                h, taps = self.target.forward_token(int(tok), p)
                full.append(taps)
        first = self._argmax(("first", 0), self.target.logits(h))
        G = np.stack([self.pdm.feature(full[p], self.n) for p in range(self.P)])
        self.pdm.run_rows(G, 0, matrix=matrix)
        self.pdm.commit(self.P)
        self.tokens = [int(x) for x in prompt] + [int(first)]
        self.reseed = (int(first), self.P)
        self.emitted = 1
        return int(first)

    # -- decisions taken in floating point, with teacher forcing ------------
    def _argmax(self, key, logits):
        y = int(np.argmax(logits))
        if self.teacher is None or key not in self.teacher or self.teacher[key] == y:
            return y
        theirs = int(self.teacher[key])
        gap = float(logits[y] - logits[theirs])
        (self.adopted if gap <= self.tol else self.mismatch).append((key, y, theirs, gap))
        return theirs

    def committed(self) -> int:
        return self.target.kv[0].length

    def inflight_positions(self) -> List[int]:
        return sorted(self.levels)

    # -- one cycle -------------------------------------------------------
    def cycle(self) -> dict:
        n, c, Wd = self.n, self.ncycles, self.Wd
        # 1. entry
        if self.reseed is not None:
            tok, t = self.reseed
            self.reseed = None
            # parent: the exited token it follows (none right after prefill)
            new = [Node(t, tok, self.pending, 0.0)]
            parents = [-1]
        else:
            t = max(self.levels) + 1
            leaves = self.levels[t - 1]
            chosen = [cd for cd in self.cands if any(cd[0] is lf for lf in leaves)][:Wd]
            chosen = self._teach_entry(c, chosen, leaves)
            new = [Node(t, tok, leaf, float(lq)) for leaf, tok, _, lq in chosen]
            parents = [next(i for i, lf in enumerate(leaves) if lf is nd.parent) for nd in new]
        for nd in new:
            nd.h = self.target.embed(nd.tok)
            nd.taps = [None] * len(self.w.anchors)
            nd.taps[0] = nd.h.copy()
        self.levels[t] = new
        # branches that got no child are dead: only the paths to the new
        # leaves stay in flight
        live = {id(x) for nd in new for x in nd.path(-1)}
        for p in self.levels:
            if p < t:
                self.levels[p] = [x for x in self.levels[p] if id(x) in live]
        if len(self.tokens) <= t:
            self.tokens.extend([-1] * (t + 1 - len(self.tokens)))
        self.tokens[t] = new[0].tok if len(new) == 1 else -1
        pos = self.inflight_positions()
        a = len(pos)
        assert 1 <= a <= n, f"occupancy {a}"
        assert pos == list(range(t - a + 1, t + 1))
        assert len(self.levels[pos[0]]) == 1, "the oldest in-flight position holds one node"
        F = self.committed()
        assert F == pos[0] or (self.pending is not None and F == pos[0]), (F, pos)
        nodes_total = sum(len(self.levels[p]) for p in pos)

        # 2. draft module (pre-step) over the tree
        pending_row = self.pending is not None
        rows = ([(self.pending, n)] if pending_row else []) + \
               [(nd, t - p) for p in pos for nd in self.levels[p]]
        # collapsed to positions, the depths are the staircase of the linear pipeline
        depth_by_pos = []
        for nd, k in rows:
            if not depth_by_pos or depth_by_pos[-1][0] != nd.pos:
                depth_by_pos.append((nd.pos, k))
        assert [k for _, k in depth_by_pos] == depth_layout(a, pending_row, n)
        cands, top_tok = self._draft(c, t, rows, commit=pending_row)
        if pending_row:
            self.pending = None

        # 3. stage step: every node through its own stage (per-branch KV)
        for p in pos:
            k = t - p
            for nd in self.levels[p]:
                self._run_stage(nd, k, F)

        # 4. exit and verification of the children
        exit_pos, y, accept, acc_rank = -1, -1, -1, -1
        if a == n:
            j = pos[0]
            nj = self.levels.pop(j)[0]
            for l in range(self.L):
                kv = self.target.kv[l]
                assert kv.length == j, (l, kv.length, j)
                kv.K[j], kv.V[j] = nj.kv[l]
                kv.length = j + 1
            lg = self.target.logits(nj.h)
            if self.hook is not None:
                self.hook("exit", dict(cycle=c, pos=j, h=nj.h, logits=lg))
            y = self._argmax(("y", c), lg)
            children = self.levels.get(j + 1, [])
            assert children and all(ch.parent is nj for ch in children)
            match = [i for i, ch in enumerate(children) if ch.tok == y]
            self.tokens[j + 1] = int(y)
            self.emitted += 1
            self.pending = nj
            exit_pos = j
            if match:
                accept, acc_rank = 1, match[0]
                self._prune_to(children[acc_rank], j)
            else:
                accept = 0
                for l in range(self.L):
                    self.target.kv[l].length = j + 1      # (i) truncate every layer
                self.levels = {}                           # (ii) flush the tree
                self.cands = []
                self.reseed = (int(y), j + 1)              # (iii) re-seed stage 0
        if accept != 0:
            self.cands = cands
        # the position that will enter next: its (unique) token once verified
        rec = dict(cycle=c, t=t, a=a, nodes=nodes_total, n_new=len(new), new_parent=parents,
                   new_token=[nd.tok for nd in new], pending_row=int(pending_row), pdm_top=int(top_tok),
                   exit_pos=exit_pos, y=int(y), accept=int(accept), acc_rank=acc_rank,
                   committed=self.committed(), pdm_len=self.pdm.C, emitted=self.emitted)
        self.logs.append(rec)
        self.ncycles += 1
        return rec

    def _prune_to(self, keep: Node, j: int) -> None:
        """After an accepted verification: only the kept child's subtree stays."""
        for p in sorted(self.levels):
            self.levels[p] = [nd for nd in self.levels[p] if keep in nd.path(j)]
            assert self.levels[p], "the kept child has a descendant at every in-flight position"

    def _run_stage(self, nd: Node, k: int, F: int) -> None:
        s = self.s
        anc = nd.path(F - 1)[:-1]  # in-flight ancestors, oldest first
        for l in stage_layers(k, self.L, self.n, s.split):
            kv = self.target.kv[l]
            Kp = np.concatenate([kv.K[:F]] + [x.kv[l][0][None] for x in anc], axis=0)
            Vp = np.concatenate([kv.V[:F]] + [x.kv[l][1][None] for x in anc], axis=0)
            nd.h, kk, vv = _step_layer(s, self.target.W["layers"][l], nd.h, nd.pos, Kp, Vp, s.bf16)
            nd.kv[l] = (kk, vv)
            if (l + 1) in self.target.anchor_at:
                nd.taps[self.target.anchor_at[l + 1]] = nd.h.copy()

    # -- the draft module over the tree -----------------------------------
    def _pdm_layers(self, G: np.ndarray, rows) -> np.ndarray:
        """Ls draft-module layers over the tree rows: row i attends to the
        committed prefix [0, C), to its ancestor rows and to itself."""
        s, pdm = self.s, self.pdm
        C = pdm.C
        X = G.astype(F32)
        idx = {id(nd): i for i, (nd, _) in enumerate(rows)}
        anc = []
        for nd, _ in rows:
            chain, x = [], nd.parent if nd.pos > C else None
            while x is not None and x.pos >= C and id(x) in idx:
                chain.append(idx[id(x)])
                x = x.parent
            if nd is not rows[0][0] and rows[0][1] == self.n and rows[0][0].pos == C and idx[id(rows[0][0])] not in chain:
                chain.append(0)  # the pending row (the exited parent of the oldest in-flight node)
            anc.append(sorted(chain, key=lambda r: rows[r][0].pos))
        for l in range(s.Ls):
            lw = pdm.W["pdm_layers"][l]
            kv = pdm.kv[l]
            Q, Ks, Vs = [], [], []
            for i, (nd, _) in enumerate(rows):
                u = rmsnorm(X[i], lw["attn_norm"], s.eps)
                q, k, v = _qkv(lw, u, s.Hq, s.Hkv, s.hd)
                cc, sn = rope_cos_sin(nd.pos, s.hd, s.base)
                q, k = apply_rope(q, cc, sn), apply_rope(k, cc, sn)
                if s.bf16:
                    from .layers import bf16_round
                    k, v = bf16_round(k), bf16_round(v)
                Q.append(q)
                Ks.append(k)
                Vs.append(v)
            out = np.empty_like(X)
            for i, (nd, _) in enumerate(rows):
                K = np.concatenate([kv.K[:C]] + [Ks[r][None] for r in anc[i]] + [Ks[i][None]], axis=0)
                V = np.concatenate([kv.V[:C]] + [Vs[r][None] for r in anc[i]] + [Vs[i][None]], axis=0)
                o = attention(Q[i], K, V)
                h = X[i] + lw["w_o"] @ o.reshape(-1)
                out[i] = _ffn(lw, h, s.F, s.eps)
            if rows and rows[0][1] == self.n and rows[0][0].pos == C:
                kv.K[C], kv.V[C] = Ks[0], Vs[0]  # the committed row's key/values stay
            X = out
        return X

    def _draft(self, c: int, t: int, rows, commit: bool):
        pdm = self.pdm
        G = np.stack([pdm.feature(nd.taps, k) for nd, k in rows])
        X = self._pdm_layers(G, rows)
        if self.hook is not None:
            self.hook("pdm_rows", dict(cycle=c, rows=rows, G=G, X=X, C=pdm.C))
        if commit:
            pdm.commit(1)
        leaves = self.levels[t]
        base = len(rows) - len(leaves)
        top_tok = -1
        cands = []
        lq_all = []
        for r, leaf in enumerate(leaves):
            lg = pdm.logits(X[base + r])
            if self.hook is not None:
                self.hook("pdm", dict(cycle=c, rank=r, leaf=leaf, logits=lg))
            lq = log_softmax64(lg)
            lq_all.append(lq)
            cum = sum(x.logq for x in leaf.path(min(self.levels)))
            order = np.lexsort((np.arange(len(lg)), -lg.astype(np.float64)))[: self.Wd]
            if r == 0:
                top_tok = int(order[0])
            for x in order:
                cands.append((leaf, int(x), cum + float(lq[x]), float(lq[x]), r))
        cands.sort(key=lambda cd: (-cd[2], cd[4], cd[1]))
        cands = [(lf, x, sc, lq) for lf, x, sc, lq, _ in cands]
        cands = self._force(t + 1, cands, leaves, lq_all)
        return cands, top_tok

    def _force(self, q: int, cands, leaves, lq_all):
        pol = self.policy
        if pol is None or q >= len(pol.ref):
            return cands
        oldest = min(self.levels)

        def matched(leaf):
            k = 0
            for x in leaf.path(oldest - 1):
                if x.tok != pol.ref[x.pos]:
                    break
                k += 1
            return k
        m = [matched(lf) for lf in leaves]
        star = m.index(max(m))
        leaf, R = leaves[star], pol.ref[q]
        u = pol.u[q, U_FORCE]
        cum = sum(x.logq for x in leaf.path(oldest))
        lq = lq_all[star]
        cands = [cd for cd in cands]
        at = [i for i, cd in enumerate(cands) if cd[0] is leaf and cd[1] == R]
        if u < pol.p1 or (u < pol.pW and self.Wd >= 2):
            if at:
                cands.pop(at[0])
            cands.insert(0 if u < pol.p1 else min(self.Wd - 1, len(cands)), (leaf, R, cum + float(lq[R]), float(lq[R])))
        else:
            def next_free():
                used = {cd[1] for cd in cands if cd[0] is leaf}
                x = (R + 1) % self.V
                while x in used:
                    x = (x + 1) % self.V
                return x
            if at:
                x = next_free()
                cands[at[0]] = (leaf, x, cum + float(lq[x]), float(lq[x]))
            if not any(cd[0] is leaf for cd in cands[: self.Wd]):
                x = next_free()
                cands.insert(min(self.Wd - 1, len(cands)), (leaf, x, cum + float(lq[x]), float(lq[x])))
        return cands

    def _teach_entry(self, c: int, chosen, leaves):
        """Adopt the teacher's entered nodes when each rank's score is within
        tol of the oracle's candidate at that rank (near-ties of the ranking)."""
        key = ("entry", c)
        if self.teacher is None or key not in self.teacher:
            return chosen
        theirs = [(int(pr), int(tk)) for pr, tk in self.teacher[key]]
        mine = [(next(i for i, lf in enumerate(leaves) if lf is cd[0]), cd[1]) for cd in chosen]
        if theirs == mine:
            return chosen
        if len(theirs) != len(mine) or any(not 0 <= pr < len(leaves) for pr, _ in theirs):
            self.mismatch.append((key, mine, theirs, float("inf")))
            return chosen
        # scores of the teacher's pairs under the oracle's draft distributions
        score = {(id(cd[0]), cd[1]): cd for cd in self.cands}
        gap = 0.0
        out = []
        for (pr, tk), mc in zip(theirs, chosen):
            leaf = leaves[pr]
            cd = score.get((id(leaf), tk))
            if cd is None:
                self.mismatch.append((key, mine, theirs, float("inf")))
                return chosen
            gap = max(gap, abs(cd[2] - mc[2]))
            out.append(cd)
        (self.adopted if gap <= self.tol else self.mismatch).append((key, mine, theirs, gap))
        return out

    def run(self, prompt: Sequence[int], G: int, max_cycles: Optional[int] = None):
        self.prefill(prompt)
        while self.emitted < G:
            if max_cycles is not None and self.ncycles >= max_cycles:
                break
            self.cycle()
        return self.tokens[: self.P + self.emitted], self.logs
