"""Integer skeleton of the SPD cycle, replayed from a run's float-decided integers.

Test infrastructure only (see the package header).

Only a few integers of a cycle are decided by floating point: the draft
module's prediction (an argmax, or a draw from Q under sampling) and, when a
token exits, the target's token (and, under sampling, the accept bit).  The
schedule fixes everything else ([RB] method steps 1-5, [PL] 3.1-3.4, [TW]
3 and 6): the newest position, the occupancy, whether the just-verified row
is pending in the draft module, the draft after the policy, which position
exits, the accept decision under greedy verification, every layer's KV
length (each token appends one entry to each layer of its stage; a rejection
truncates all layers to j+1), the draft module's committed length and the
emitted count.  `Replay` recomputes those from the decided integers alone, so
a recorded run of any size can be checked field by field.  It also tracks the
tokens in flight, which tells which cycles' draft-module inputs are made of
finally-verified tokens only.

Readings are those of the full state machine: the exiting token j verifies
j+1, a rejection truncates to j+1 and re-seeds (y, j+1), the just-verified row
is committed in the cycle after its exit -- or, under the post-step schedule
(the scheduling ablation of [PL] §4), in the cycle of its exit.
"""
from __future__ import annotations

from typing import Dict, List, Optional

from .schedule import stage_layers


class ReplayError(AssertionError):
    pass


class Replay:
    def __init__(self, n: int, L: int, P: int, first: int, policy=None, sample: bool = False,
                 post: bool = False, split=()):
        if not split and L % n:
            raise ValueError("n must divide L")
        self.n, self.L = n, L
        self.layers = [stage_layers(k, L, n, split) for k in range(n)]
        self.policy = policy
        self.sample = sample
        self.post = post
        self.kv: List[int] = [P] * L
        self.C = P
        self.pending = False
        self.inflight: List[list] = []            # [pos, depth, token], oldest first
        self.drafts: Dict[int, tuple] = {}         # pos -> (token, drafting cycle)
        self.tokens: Dict[int, int] = {P: int(first)}
        self.seed = (int(first), P)
        self.emitted = 1
        self.c = 0

    def step(self, raw: int, y: Optional[int] = None, accepted: Optional[int] = None) -> dict:
        """One cycle.  `raw` = the draft module's prediction; `y` (and, under
        sampling, `accepted`) are required exactly when a token exits."""
        n = self.n
        tok, t = self.seed
        self.tokens[t] = tok
        self.inflight.append([t, 0, tok])
        a = len(self.inflight)
        if not 1 <= a <= n:
            raise ReplayError(f"cycle {self.c}: occupancy {a}")
        pending_row = self.pending
        row0 = self.C
        inflight_tokens = [(p, tk) for p, _, tk in self.inflight]
        if pending_row:
            self.C += 1
            self.pending = False
        if row0 != t + 1 - a - int(pending_row):
            raise ReplayError(f"cycle {self.c}: trailing rows {row0}..{t} do not match occupancy {a}")
        raw = int(raw)
        d = raw if (self.sample or self.policy is None) else int(self.policy.draft(t + 1, raw))
        self.drafts[t + 1] = (d, self.c)

        # stage step: every in-flight token appends one KV entry to each layer of its stage
        for item in self.inflight:
            p, k, _ = item
            for l in self.layers[k]:
                if self.kv[l] != p:
                    raise ReplayError(f"cycle {self.c}: layer {l} holds {self.kv[l]} entries before position {p}")
                self.kv[l] = p + 1
            item[1] = k + 1

        exit_pos, yy, acc = -1, -1, -1
        drafted_at = -1
        if self.inflight[0][1] == n:
            if y is None:
                raise ReplayError(f"cycle {self.c}: a token exits but no target token was given")
            j = self.inflight.pop(0)[0]
            xd, drafted_at = self.drafts.pop(j + 1)
            yy = int(y)
            if self.sample:
                if accepted is None:
                    raise ReplayError(f"cycle {self.c}: sampling needs the accept bit")
                acc = int(bool(accepted) and yy == xd)
                if bool(accepted) and yy != xd:
                    raise ReplayError(f"cycle {self.c}: accepted draft {xd} but emitted {yy}")
            else:
                acc = int(xd == yy)
            self.tokens[j + 1] = yy
            self.emitted += 1
            if self.post:
                self.C += 1  # committed by this cycle's (post-step) draft step
            else:
                self.pending = True
            exit_pos = j
            if not acc:
                self.kv = [j + 1] * self.L
                self.inflight = []
                self.drafts = {p: v for p, v in self.drafts.items() if p <= j}
                self.tokens = {p: v for p, v in self.tokens.items() if p <= j + 1}
                self.seed = (yy, j + 1)
        if exit_pos < 0 or acc:
            self.seed = (d, t + 1)
        rec = dict(cycle=self.c, t=t, a=a, pending_row=int(pending_row), row0=row0, pdm_raw=raw, draft=d,
                   exit_pos=exit_pos, y=yy, accept=acc, kv_len=list(self.kv), pdm_len=self.C,
                   emitted=self.emitted, inflight_tokens=inflight_tokens, drafted_at=drafted_at)
        self.c += 1
        return rec
