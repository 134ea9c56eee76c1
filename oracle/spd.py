"""The SPD cycle as a step-by-step state machine (test infrastructure only).

One cycle ([RB] method steps 1-5, [PL] §3.1-3.4, [TW] §3-6):
  1. entry: the seed token (a draft, or the corrected token after a
     rejection) enters stage 0 at depth 0;
  2. draft (pre-step): the PDM reads the features of the trailing positions
     as they stand before this cycle's stage step -- the just-verified
     position at depth n (its full-depth feature is then cached, [PL] §A.1),
     then the in-flight tokens at depths a-1..0 -- and predicts the token
     after the newest one;
  3. stage step: every in-flight token advances through the L/n layers of
     its own stage;
  4. exit: the token that completed stage n-1 produces full-depth logits that
     verify its successor (drafted about n cycles earlier);
  5. on rejection, the three-step rollback: every layer's KV cache is
     truncated to the verified length, the in-flight states are dropped, and
     stage 0 is re-seeded with the corrected token.

Post-step schedule (the scheduling ablation of [PL] §4): step 2 moves after
step 4 and reads the features as the stage step left them -- the exited
token at depth n (its draft-module key/values committed in the same cycle),
the in-flight tokens at depths a-1..1 -- so drafting waits for the stage step.
Which token enters the pipeline in each cycle follows the same rules.

Readings taken where the pages leave a step open:
  * positions are 0-indexed: the exiting token j keeps its KV, so the
    truncation length is j+1 (the pages' 1-indexed "t-n+1");
  * the exiting token verifies position j+1, the oldest draft in flight;
  * prefill is a full target pass over the prompt; the first new token comes
    from the target itself; the PDM is prefilled on the prompt's full-depth
    features; the pipeline then starts empty, seeded with that token;
  * greedy ties go to the lowest token id.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import numpy as np

from seeded_inputs import U_ACCEPT, U_DRAFT, U_FORCE, U_RESAMPLE, U_TARGET

from . import sampling
from .model import PDM, Target
from .schedule import depth_layout, key_depth, post_depth_layout


class NaturalPolicy:
    """Draft = the PDM's own prediction."""

    def draft(self, q: int, pdm_tok: int) -> int:
        return pdm_tok


class ForcedPolicy:
    """Seeded forced acceptance: a harness device for random-init draft modules.

    Not on the pages (an untrained PDM is almost never right).  When drafting
    position q < len(ref): if u[q, FORCE] < p, the draft is ref[q] (the
    target's own greedy token); otherwise it is the PDM's prediction, or
    (ref[q]+1) mod V should that happen to equal ref[q].  Positions beyond
    `ref` use the PDM's prediction.  Verification is untouched, so the output
    stays the target's greedy output whatever the policy.
    """

    def __init__(self, ref: Sequence[int], p_accept: float, uniforms: np.ndarray, V: int):
        self.ref = np.asarray(ref, dtype=np.int64)
        self.p = np.float32(p_accept)
        self.u = uniforms
        self.V = V

    def draft(self, q: int, pdm_tok: int) -> int:
        if q >= len(self.ref):
            return pdm_tok
        r = int(self.ref[q])
        if self.u[q, U_FORCE] < self.p:
            return r
        return pdm_tok if pdm_tok != r else (r + 1) % self.V


class FixedPolicy:
    """Draft = ref[q] where right[q] is set, else a token != ref[q] (test policy)."""

    def __init__(self, ref: Sequence[int], right: Sequence[bool], V: int):
        self.ref, self.right, self.V = list(ref), list(right), V

    def draft(self, q: int, pdm_tok: int) -> int:
        if q >= len(self.ref):
            return pdm_tok
        r = self.ref[q]
        if self.right[q]:
            return r
        return pdm_tok if pdm_tok != r else (r + 1) % self.V


class Decisions:
    """Integer decisions taken from floating point, with optional teacher forcing.

    Greedy argmax picks the lowest id among equal maxima.  With a teacher (the
    decisions another implementation took, keyed by (kind, cycle)), a differing
    choice is adopted when it is also valid within `tol` -- a logit within tol
    of the maximum (`tol`, logit units), a top-k kept set whose excluded ids
    beat no kept id by more than tol, or a sampling threshold within
    `sample_tol` of the boundary it falls on (as a fraction of the total mass,
    or for the accept test of Q(x)) -- and recorded; otherwise it is recorded
    as a mismatch.  Without a teacher nothing is adopted.
    """

    def __init__(self, teacher: Optional[Dict] = None, tol: float = 0.0, sample_tol: Optional[float] = None):
        self.teacher = teacher
        self.tol = tol
        self.sample_tol = tol if sample_tol is None else sample_tol
        self.adopted: List[tuple] = []
        self.mismatch: List[tuple] = []

    def _teach(self, key, mine, valid_fn, tol):
        if self.teacher is None or key not in self.teacher:
            return mine
        theirs = self.teacher[key]
        if theirs == mine:
            return mine
        gap = valid_fn(theirs)
        rec = (key, mine, theirs, gap)
        (self.adopted if gap <= tol else self.mismatch).append(rec)
        return theirs

    def argmax(self, key, logits: np.ndarray) -> int:
        y = int(np.argmax(logits))
        return self._teach(key, y, lambda t: float(logits[y] - logits[t]), self.tol)

    def kept_set(self, key, logits: np.ndarray, k: int) -> np.ndarray:
        """Top-k kept ids (ascending) of `logits`; a teacher's set replaces the
        oracle's when it is a valid top-k choice within `tol`."""
        mine = sampling.top_k_ids(logits, k)
        if self.teacher is None or key not in self.teacher:
            return mine
        theirs = np.sort(np.asarray(self.teacher[key], np.int64))
        if len(theirs) == len(mine) and np.array_equal(theirs, mine):
            return mine
        ok_size = len(theirs) == len(mine) and len(np.unique(theirs)) == len(theirs) and \
            theirs.min() >= 0 and theirs.max() < len(logits)
        gap = sampling.top_k_set_gap(logits, theirs) if ok_size else float("inf")
        rec = (key, "set", len(np.setdiff1d(theirs, mine)), gap)
        (self.adopted if gap <= self.tol else self.mismatch).append(rec)
        return theirs if ok_size else mine

    def sample(self, key, weights: np.ndarray, u: float, tol: Optional[float] = None) -> int:
        """A draw by inverse CDF; a differing teacher draw must lie within
        `sample_tol` (or `tol`; fraction of the total mass) of its interval."""
        i, _ = sampling.inverse_cdf(weights, u)
        c = np.cumsum(weights.astype(np.float64))
        thr = np.float64(u) * c[-1]

        def gap(t):
            if not 0 <= t < len(c):
                return float("inf")
            lo = c[t - 1] if t > 0 else 0.0
            return float(max(lo - thr, thr - c[t], 0.0) / c[-1])
        return self._teach(key, i, gap, self.sample_tol if tol is None else tol)

    def accept(self, key, p_w, p_Z, q_w, q_Z, x, u, tol: Optional[float] = None) -> bool:
        acc, g = sampling.accept_test(p_w, p_Z, q_w, q_Z, x, u)
        return bool(self._teach(key, acc, lambda t: g, self.sample_tol if tol is None else tol))


class SPDOracle:
    """Runs prefill and SPD cycles, logging every cycle's integer state."""

    def __init__(self, w, W, policy=None, uniforms: Optional[np.ndarray] = None,
                 teacher: Optional[Dict] = None, tol: float = 0.0, sample_tol: Optional[float] = None):
        self.w = w
        self.n, self.L, self.V = w.n, w.L, w.V
        self.target = Target(w, W)
        self.pdm = PDM(w, W)
        self.sample = w.mode == "sample"
        self.post = getattr(w, "schedule", "pre") == "post"
        if self.post and w.n < 2:
            raise ValueError("the post-step schedule needs n >= 2: with one stage the draft "
                             "would come after its own verification")
        self.T = w.temperature
        self.top_k = getattr(w, "top_k", 0)
        self.policy = policy or NaturalPolicy()
        self.u = uniforms
        if self.sample:
            assert uniforms is not None, "sampling needs the uniform table"
        self.dec = Decisions(teacher, tol, sample_tol)
        self.tokens: List[int] = []
        self.inflight: List[list] = []      # [pos, depth, h], oldest first
        self.anchors: Dict[int, list] = {}  # pos -> [h^(b_i) or None]
        self.drafts: Dict[int, tuple] = {}  # pos -> (token, (q_w, q_Z) or None)
        self.pending: Optional[int] = None  # verified position whose g_n is not cached yet
        self.seed = None
        self.emitted = 0
        self.ncycles = 0
        self.logs: List[dict] = []
        self.P = 0
        self.hook = None  # optional callable(kind, info) for inspection in tests

    # -- prefill -------------------------------------------------------------
    def prefill(self, prompt: Sequence[int], matrix: bool = False) -> int:
        """matrix=True runs the same prefill with matrix products (long prompts)."""
        n = self.n
        self.P = len(prompt)
        full = []
        h = None
        if matrix:
            h, full = self.target.prefill_matrix([int(t) for t in prompt])
        else:
            for p, tok in enumerate(prompt):
                h, taps = self.target.forward_token(int(tok), p)
                full.append(taps)
        lg = self.target.logits(h)
        if self.sample:
            pw, _ = sampling.softmax_weights(lg, self.T, keep=self._keep(("pset_first", 0), lg))
            first = self.dec.sample(("first", 0), pw, float(self.u[self.P, U_TARGET]))
        else:
            first = self.dec.argmax(("first", 0), lg)
        G = np.stack([self.pdm.feature(full[p], n) for p in range(self.P)])
        self.pdm.run_rows(G, 0, matrix=matrix)
        self.pdm.commit(self.P)
        self.tokens = [int(x) for x in prompt] + [int(first)]
        self.seed = (int(first), self.P)
        self.emitted = 1
        return int(first)

    # -- one cycle ---------------------------------------------------------
    def cycle(self) -> dict:
        n, c = self.n, self.ncycles
        tok, t = self.seed
        # 1. entry
        if len(self.tokens) <= t:
            self.tokens.extend([-1] * (t + 1 - len(self.tokens)))
        self.tokens[t] = tok
        h0 = self.target.embed(tok)
        taps = [None] * len(self.w.anchors)
        taps[0] = h0.copy()
        self.anchors[t] = taps
        self.inflight.append([t, 0, h0])
        a = len(self.inflight)
        assert 1 <= a <= n, f"occupancy {a} outside 1..{n}"
        pending_row = self.pending is not None
        post = self.post

        # 2. draft module, on the pre-step features (post-step: after step 4)
        if not post:
            rows = ([(self.pending, n)] if pending_row else []) + [(p, k) for p, k, _ in self.inflight]
            depths = [k for _, k in rows]
            assert depths == depth_layout(a, pending_row, n), (depths, a)
            for p, k in rows:
                assert key_depth(t, p, a, n) == k
            d_raw, d = self._draft(c, t, rows, commit=pending_row)
            if pending_row:
                self.anchors.pop(self.pending, None)
                self.pending = None

        # 3. stage step: each token through its own stage
        for item in self.inflight:
            p, k, h = item
            item[2] = self.target.run_stage(h, p, k, taps=self.anchors[p])
            item[1] = k + 1

        # 4. exit and streaming verification
        exit_pos, y, accept = -1, -1, -1
        if self.inflight[0][1] == n:
            j, _, hj = self.inflight.pop(0)
            lg = self.target.logits(hj)
            if self.hook is not None:
                self.hook("exit", dict(cycle=c, pos=j, h=hj, logits=lg))
            assert (j + 1) in self.drafts, "successor of an exiting token must be a draft"
            xd, qinfo = self.drafts.pop(j + 1)
            if self.sample:
                pw, pZ = sampling.softmax_weights(lg, self.T, keep=self._keep(("pset", c), lg))
                ok = self.dec.accept(("accept", c), pw, pZ, qinfo[0], qinfo[1], xd,
                                     float(self.u[j + 1, U_ACCEPT]))
                if ok:
                    y = xd
                else:
                    r = sampling.residual(pw, pZ, qinfo[0], qinfo[1])
                    y = self.dec.sample(("resample", c), r, float(self.u[j + 1, U_RESAMPLE]))
                accept = int(ok)
            else:
                y = self.dec.argmax(("y", c), lg)
                accept = int(xd == y)
            if len(self.tokens) <= j + 1:  # n = 1: the successor was drafted this cycle
                self.tokens.extend([-1] * (j + 2 - len(self.tokens)))
            self.tokens[j + 1] = int(y)
            self.emitted += 1
            if not post:
                self.pending = j
            exit_pos = j

        # 2'. post-step schedule: the draft module reads the features after
        # the stage step -- the exited token at depth n (committed now), the
        # in-flight tokens at depths a-1..1 -- and runs before the rollback
        # (a flushed cycle's draft is discarded like any other)
        if post:
            rows = ([(exit_pos, n)] if exit_pos >= 0 else []) + [(p, k) for p, k, _ in self.inflight]
            depths = [k for _, k in rows]
            assert depths == post_depth_layout(a, n), (depths, a)
            for p, k in rows:
                assert min(n, key_depth(t, p, a, n) + 1) == k
            d_raw, d = self._draft(c, t, rows, commit=exit_pos >= 0)
            if exit_pos >= 0:
                self.anchors.pop(exit_pos, None)
                self.pending = None

        # 5. transition / three-step rollback
        if exit_pos >= 0 and not accept:
            j = exit_pos
            self.target.truncate(j + 1)          # (i) every layer's KV to length j+1
            self.inflight = []                   # (ii) flush in-flight states
            for p in [p for p in self.anchors if p > j]:
                del self.anchors[p]
            for p in [p for p in self.drafts if p > j]:
                del self.drafts[p]
            self.seed = (int(y), j + 1)          # (iii) re-seed stage 0
        else:
            self.seed = (int(d), t + 1)

        rec = dict(cycle=c, t=t, a=a, pending_row=int(pending_row), depths=depths,
                   pdm_raw=int(d_raw), draft=int(d), exit_pos=exit_pos, y=int(y),
                   accept=int(accept), kv_len=[kv.length for kv in self.target.kv],
                   pdm_len=self.pdm.C, emitted=self.emitted)
        self.logs.append(rec)
        self.ncycles += 1
        return rec

    def _keep(self, key, logits):
        """Kept ids of a top-k truncated distribution (None: the whole vocabulary)."""
        if not 0 < self.top_k < self.V:
            return None
        return self.dec.kept_set(key, logits, self.top_k)

    def _draft(self, c: int, t: int, rows, commit: bool):
        """Draft-module step over the trailing rows [(position, depth)]: the
        features g(p, k), the Ls layers over committed + trailing rows, the
        first row's key/values committed if `commit`, and the prediction for
        position t+1 from the newest row ([RB] method steps 2-4)."""
        positions = [p for p, _ in rows]
        assert positions == list(range(self.pdm.C, t + 1)), (positions, self.pdm.C)
        Gm = np.stack([self.pdm.feature(self.anchors[p], k) for p, k in rows])
        X = self.pdm.run_rows(Gm, self.pdm.C)
        if commit:
            self.pdm.commit(1)
        pl = self.pdm.logits(X[-1])
        if self.hook is not None:
            self.hook("pdm", dict(cycle=c, rows=rows, G=Gm, X=X, logits=pl))
        if self.sample:
            qw, qZ = sampling.softmax_weights(pl, self.T, keep=self._keep(("qset", c), pl))
            d_raw = self.dec.sample(("draft", c), qw, float(self.u[t + 1, U_DRAFT]))
            d = d_raw
            self.drafts[t + 1] = (d, (qw, qZ))
        else:
            d_raw = self.dec.argmax(("pdm", c), pl)
            d = int(self.policy.draft(t + 1, d_raw))
            self.drafts[t + 1] = (d, None)
        return d_raw, d

    def run(self, prompt: Sequence[int], G: int, max_cycles: Optional[int] = None):
        """Prefill, then cycle until G tokens are emitted (the first from prefill)."""
        self.prefill(prompt)
        while self.emitted < G:
            if max_cycles is not None and self.ncycles >= max_cycles:
                break
            self.cycle()
        return self.tokens[: self.P + self.emitted], self.logs


def ar_continue(o: "SPDOracle", n_tokens: int) -> List[int]:
    """Greedy AR continuation from a prefilled oracle's state (its KV copied).

    Returns the token list of positions 0 .. P + n_tokens (prompt, the
    prefill token and n_tokens more).
    """
    import copy

    tgt = copy.deepcopy(o.target)
    toks = list(o.tokens[: o.P + 1])
    while len(toks) < o.P + 1 + n_tokens:
        h, _ = tgt.forward_token(toks[-1], len(toks) - 1)
        toks.append(int(np.argmax(tgt.logits(h))))
    return toks


def ar_greedy(w, W, prompt: Sequence[int], G: int):
    """Plain greedy autoregressive decoding of the target: the lossless reference.

    Returns (tokens of prompt + G new tokens, the Target with its KV caches).
    """
    tgt = Target(w, W)
    h = None
    for p, tok in enumerate(prompt):
        h, _ = tgt.forward_token(int(tok), p)
    toks = [int(x) for x in prompt]
    toks.append(int(np.argmax(tgt.logits(h))))
    while len(toks) < len(prompt) + G:
        h, _ = tgt.forward_token(toks[-1], len(toks) - 1)
        toks.append(int(np.argmax(tgt.logits(h))))
    return toks, tgt
