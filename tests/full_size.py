"""Full-size runs of the HIP path and the oracle checks that scale to them.

A full-size generation is too long for the oracle to run cycle by cycle, so
it is checked in pieces that together cover every integer a cycle produces,
plus floating-point state at two stopping points:

1. integer replay (oracle.replay) of every cycle from the integers that
   floating point decided; under greedy decoding the output must also equal
   the GPU's own autoregressive decode (losslessness holds at any size);
2. every verification: one oracle target forward (matrix form) over the
   final sequence gives the logits at every exiting position, so the target
   token of every exit is compared with the oracle's argmax (a differing
   choice must be a near-tie: its oracle logit within the tolerance of the
   maximum);
3. the draft module at sampled cycles whose in-flight tokens all survived
   (so that the forward's anchors are theirs): the oracle rebuilds the
   trailing rows' features at their depths, runs its layers over the
   committed prefix (one matrix pass over every position's full-depth
   feature) plus those rows, and its head.  Under sampling, EVERY
   verification recomputes Q at the cycle that drafted the verified position
   and retakes the draw, the accept test and the residual redraw with the
   same seeded uniforms.  Under top-k, the kept sets the GPU used (the top-k
   ids of its own logits, read back in a second, cycle-by-cycle generation
   that must reproduce the first bit for bit) must be valid top-k choices of
   the oracle's logits, and the draws are retaken on those sets.

The GPU side runs exactly as the benchmark times it: weights generated on the
device, graph-launched cycles, the forced-acceptance reference from the
GPU's own autoregressive decode.
"""
from __future__ import annotations

import numpy as np

import seeded_inputs as si
from oracle import sampling, schedule
from oracle.model import PDM, Target
from oracle.replay import Replay
from oracle.spd import Decisions, ForcedPolicy
from seeded_inputs import U_ACCEPT, U_DRAFT, U_RESAMPLE, U_TARGET

IDLE = 8  # record flag of a cycle enqueued after the generation ended
TOL = {"f32": 1e-4, "bf16": 0.05}       # near-tie margin of an argmax (logit units)
STOL = {"f32": 1e-5, "bf16": 2e-4}      # near-tie of a draw (fraction of the mass)
RTOL = {"f32": 1e-4, "bf16": 2e-2}      # rel-L2 of hidden states, anchors, logits, KV
INT_FIELDS = [("t", "t"), ("occupancy", "a"), ("pending_row", "pending_row"), ("draft", "draft"),
              ("exit_pos", "exit_pos"), ("target_token", "y"), ("accepted", "accept"),
              ("pdm_len", "pdm_len"), ("emitted", "emitted")]


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


def _snapshot(eng, recs):
    last = recs[-1]
    t, a = int(last["t"]), int(last["occupancy"])
    snap = dict(index=len(recs) - 1, pdm_logits=eng.pdm_logits(),
                anchors={p: eng.anchors(p) for p in range(t - a + 1, t + 1)})
    ex = np.flatnonzero(recs["exit_pos"] >= 0)
    if len(ex):
        snap["exit_index"] = int(ex[-1])
        snap["logits"] = eng.logits()
    return snap


def gpu_run(name: str) -> dict:
    """One full generation of workload `name` on cuda:0 (graph launch mode)."""
    import torch
    from pipelined_draft_verify_amd import SPDEngine

    w = si.workload(name)
    T = si.make_weights(w, "cuda:0")
    eng = SPDEngine(w, T)
    eng.set_launch_mode(True)
    uni = si.make_uniforms(w)
    eng.set_uniforms(uni)
    prompt = si.make_prompt(w)
    first = int(eng.prefill(prompt))
    first_set = None
    if w.mode == "sample" and w.top_k:
        from oracle.sampling import top_k_ids
        lg = eng.logits()  # the prefill's logits
        first_set = top_k_ids(lg, w.top_k)
        first_val = lg[first_set].copy()
    ref = None
    if w.mode == "greedy":
        ar = eng.generate_ar(w.G - 1)
        ref = [int(x) for x in prompt] + [first] + [int(x) for x in ar]
        eng.rollback(w.P, first)
        if w.policy == "forced":
            eng.set_forced(ref, w.p_accept)
    k0 = 3 * w.n + 2
    buf = eng.enqueue(k0)
    eng.sync()
    head = eng.records_of(buf)
    head = head[(head["flags"] & IDLE) == 0]
    mid = _snapshot(eng, head)
    rest = eng.run(batch=256)
    recs = np.concatenate([head, rest])
    toks = eng.tokens(0, w.P + w.G)
    end = _snapshot(eng, recs)
    end["kv"] = {l: (eng.kv(l, "k"), eng.kv(l, "v")) for l in sorted({0, w.L // 2, w.L - 1})}
    sets = None
    if first_set is not None:
        sets = _topk_sets(eng, w, first, recs)
        sets[("pset_first", 0)] = first_set
        sets[("pval_first", 0)] = first_val
    elif w.mode == "sample":
        sets = _dense_logs(eng, w, first, recs)
    eng.close()
    del eng
    flat = si.weights_numpy_f32(T)
    del T
    torch.cuda.empty_cache()
    return dict(w=w, W=si.nest_weights(flat, w), prompt=prompt, uni=uni, first=first, ref=ref,
                recs=recs, toks=[int(x) for x in toks], mid=mid, end=end, sets=sets)


def _topk_sets(eng, w, first, recs):
    """The generation again, one cycle at a time, reading the logits behind
    every top-k truncation: the kept sets (top-k ids of the GPU's logits,
    ties to the lower id) and the GPU's logits at those ids.  Its records
    must equal the first run's."""
    from oracle.sampling import top_k_ids

    eng.rollback(w.P, first)
    sets = {}
    out = []
    while True:
        buf = eng.enqueue(1)
        st = eng.sync()
        r = eng.records_of(buf)
        if r["flags"][0] & IDLE:
            break
        c = len(out)
        ql = eng.pdm_logits()
        sets[("qset", c)] = top_k_ids(ql, w.top_k)
        sets[("qval", c)] = ql[sets[("qset", c)]].copy()
        if r["exit_pos"][0] >= 0:
            pl = eng.logits()
            sets[("pset", c)] = top_k_ids(pl, w.top_k)
            sets[("pval", c)] = pl[sets[("pset", c)]].copy()
        out.append(r)
        if st.done:
            break
    again = np.concatenate(out)
    a, b = recs.copy(), again.copy()
    a["cycle"] -= a["cycle"][0]
    b["cycle"] -= b["cycle"][0]
    assert a.tobytes() == b.tobytes(), "cycle-by-cycle generation differs from the graph-launched one"
    return sets


def _log_softmax64(l: np.ndarray, T: float) -> np.ndarray:
    x = l.astype(np.float64) / T
    m = x.max()
    return x - m - np.log(np.sum(np.exp(x - m)))


def _dense_logs(eng, w, first, recs):
    """Dense sampling: the generation again, one cycle at a time, reading the
    GPU's own log Q(x) of every cycle's draft x (from its draft logits) and
    the log-softmax of its target logits at every exit (kept as the logits),
    for the accept tests.  Its records must equal the first run's."""
    eng.rollback(w.P, first)
    logs = {}
    out = []
    while True:
        buf = eng.enqueue(1)
        st = eng.sync()
        r = eng.records_of(buf)
        if r["flags"][0] & IDLE:
            break
        c = len(out)
        x = int(r["draft"][0])
        if x >= 0:
            logs[("qlog", c)] = float(_log_softmax64(eng.pdm_logits(), w.temperature)[x])
        if r["exit_pos"][0] >= 0:
            logs[("plogits", c)] = eng.logits().copy()
        out.append(r)
        if st.done:
            break
    again = np.concatenate(out)
    a, b = recs.copy(), again.copy()
    a["cycle"] -= a["cycle"][0]
    b["cycle"] -= b["cycle"][0]
    assert a.tobytes() == b.tobytes(), "cycle-by-cycle generation differs from the graph-launched one"
    return logs


def replay(run: dict):
    """Integer replay of every cycle; returns the replay records."""
    w, recs = run["w"], run["recs"]
    pol = None
    if w.mode == "greedy" and w.policy == "forced":
        pol = ForcedPolicy(run["ref"], w.p_accept, run["uni"], w.V)
    rp = Replay(w.n, w.L, w.P, run["first"], policy=pol, sample=(w.mode == "sample"),
                post=(w.schedule == "post"), split=w.split)
    out = []
    for i, r in enumerate(recs):
        ex = int(r["exit_pos"]) >= 0
        q = rp.step(int(r["pdm_argmax"]), int(r["target_token"]) if ex else None,
                    int(r["accepted"]) if ex else None)
        for gf, of in INT_FIELDS:
            assert int(r[gf]) == q[of], (i, gf, int(r[gf]), q[of])
        assert list(map(int, r["kv_len"][: w.L])) == q["kv_len"], (i, "kv_len")
        assert int(r["flags"]) == 0, (i, "flags", int(r["flags"]))
        out.append(q)
    return out, rp


class OracleView:
    """The oracle's target forward over the final sequence and the draft
    module's KV over every position's full-depth feature."""

    def __init__(self, run: dict):
        w, W = run["w"], run["W"]
        self.w = w
        self.toks = run["toks"]
        self.N = w.P + w.G - 1  # positions 0 .. P+G-2: every exiting position
        self.tgt = Target(w, W)
        H, self.taps = self.tgt.prefill_matrix(self.toks[: self.N], all_rows=True)
        self.LG = self.tgt.logits_rows(H[w.P - 1:])
        del H
        self.pdm = PDM(w, W)
        self.pdm.run_rows(self.pdm.feature_rows(self.taps, w.n), 0, matrix=True)

    def logits_at(self, j: int) -> np.ndarray:
        return self.LG[j - (self.w.P - 1)]

    def survived(self, q: dict, upto: int = None) -> bool:
        """All in-flight tokens of replay record q (at positions <= upto) are final."""
        return all(p < self.N and self.toks[p] == tk for p, tk in q["inflight_tokens"]
                   if upto is None or p <= upto)

    def pdm_logits(self, q: dict) -> np.ndarray:
        """Draft-module logits of the cycle of replay record q (rows row0..t)."""
        return self.pdm.logits(self.pdm_last_row(q))

    def pdm_head_rows(self, X: np.ndarray) -> np.ndarray:
        """The draft head over many final rows at once: [M, V]."""
        from oracle.layers import rmsnorm
        W = self.pdm.W
        U = np.stack([rmsnorm(x, W["pdm_final_norm"], self.w.eps) for x in X])
        return (U @ W["pdm_lm_head"].T).astype(np.float32)

    def pdm_last_row(self, q: dict) -> np.ndarray:
        """Final draft-module row (before the head) of the cycle of replay record q."""
        w, pdm = self.w, self.pdm
        row0, t = q["row0"], q["t"]
        if w.schedule == "post":
            depths = schedule.post_depth_layout(q["a"], w.n)
        else:
            depths = schedule.depth_layout(q["a"], bool(q["pending_row"]), w.n)
        G = np.stack([pdm.feature(self.taps[p], k) for p, k in zip(range(row0, t + 1), depths)])
        saved = [(kv.K[row0:t + 1].copy(), kv.V[row0:t + 1].copy()) for kv in pdm.kv]
        C0 = pdm.C
        pdm.C = row0
        try:
            X = pdm.run_rows(G, row0, matrix=True)
        finally:
            pdm.C = C0
            for kv, (K, V) in zip(pdm.kv, saved):
                kv.K[row0:t + 1] = K
                kv.V[row0:t + 1] = V
        return X[-1]


def check_verifications(run: dict, view: OracleView, reps) -> Decisions:
    """Greedy: the first token and the target token of every exit."""
    w, recs = run["w"], run["recs"]
    teacher = {("first", 0): run["first"]}
    dec = Decisions(teacher, TOL[w.dtype])
    dec.argmax(("first", 0), view.logits_at(w.P - 1))
    for i, r in enumerate(recs):
        if int(r["exit_pos"]) < 0:
            continue
        teacher[("y", i)] = int(r["target_token"])
        dec.argmax(("y", i), view.logits_at(int(r["exit_pos"])))
    return dec


def sample_indices(cands, k: int):
    cands = list(cands)
    if len(cands) <= k:
        return cands
    return sorted({cands[int(round(x))] for x in np.linspace(0, len(cands) - 1, k)})


def check_draft_module(run: dict, view: OracleView, reps, k: int = 32) -> Decisions:
    """Greedy: the draft module's argmax at sampled cycles whose inputs survived."""
    w, recs = run["w"], run["recs"]
    cands = [i for i, q in enumerate(reps) if q["t"] < view.N and view.survived(q)]
    assert len(cands) >= min(k, 8), len(cands)
    teacher = {}
    dec = Decisions(teacher, TOL[w.dtype])
    for i in sample_indices(cands, k):
        teacher[("pdm", i)] = int(recs[i]["pdm_argmax"])
        dec.argmax(("pdm", i), view.pdm_logits(reps[i]))
    dec.checked = len(sample_indices(cands, k))
    return dec


def _on_set(V: int, ids, vals) -> np.ndarray:
    """A logits vector holding `vals` at `ids` and -inf elsewhere."""
    out = np.full(V, -np.inf, np.float32)
    out[np.asarray(ids, np.int64)] = vals
    return out


def check_sampling(run: dict, view: OracleView, reps, chunk: int = 32, progress=None) -> Decisions:
    """Sampling: the first token, and at EVERY verification the draft draw
    from Q (recomputed at the cycle that drafted the verified position), the
    accept test u*Q(x) < P(x) and the residual redraw.

    Dense (whole-vocabulary) distributions: a differing decision must lie
    within STOL of its boundary in the oracle's arithmetic.

    Top-k: the GPU's kept sets and its logits at them come in from the
    cycle-by-cycle run.  Each set must be a valid top-k choice of the
    oracle's logits (argmax tolerance), the GPU's logits at its set must be
    within the argmax tolerance of the oracle's, every decision retaken on
    the GPU's own logits must reproduce the GPU's decision (the sampler's
    arithmetic; 1e-6 of the mass for rounding), and retaken on the oracle's
    logits over the same set it may differ only within the shift that the
    measured logit difference allows (oracle.sampling *_shift_bound)."""
    w, recs, uni = run["w"], run["recs"], run["uni"]
    T, k = w.temperature, w.top_k
    topk = 0 < k < w.V
    teacher = dict(run.get("sets") or {})
    teacher[("first", 0)] = run["first"]
    dec = Decisions(teacher, TOL[w.dtype], STOL[w.dtype])
    own = Decisions(teacher, TOL[w.dtype], 1e-6)  # decisions retaken on the GPU's own logits
    dec.eps = 0.0

    def eps_of(sk, vk, logits):
        """Largest difference of the GPU's and the oracle's logits on the GPU's set."""
        e = float(np.max(np.abs(np.asarray(teacher[vk], np.float64) - logits[teacher[sk]])))
        dec.eps = max(dec.eps, e)
        if e > TOL[w.dtype]:
            dec.mismatch.append((vk, "logits", e))
        return e

    l0 = view.logits_at(w.P - 1)
    if topk:
        S0 = dec.kept_set(("pset_first", 0), l0, k)
        e0 = eps_of(("pset_first", 0), ("pval_first", 0), l0)
        gw0, _ = sampling.softmax_weights(_on_set(w.V, teacher[("pset_first", 0)], teacher[("pval_first", 0)]), T,
                                          keep=teacher[("pset_first", 0)])
        own.sample(("first", 0), gw0, float(uni[w.P, U_TARGET]))
        pw0, _ = sampling.softmax_weights(l0, T, keep=S0)
        dec.sample(("first", 0), pw0, float(uni[w.P, U_TARGET]),
                   tol=max(STOL[w.dtype], sampling.cdf_shift_bound(e0, T)))
    else:
        pw0, _ = sampling.softmax_weights(l0, T)
        dec.sample(("first", 0), pw0, float(uni[w.P, U_TARGET]))
    exits = [i for i, q in enumerate(reps) if q["exit_pos"] >= 0]
    for b0 in range(0, len(exits), chunk):
        batch = exits[b0:b0 + chunk]
        rows = []
        for i in batch:
            qd = reps[reps[i]["drafted_at"]]
            assert qd["t"] == reps[i]["exit_pos"] and view.survived(qd)
            rows.append(view.pdm_last_row(qd))
        QL = view.pdm_head_rows(np.stack(rows))
        for i, ql in zip(batch, QL):
            q = reps[i]
            j, c2 = q["exit_pos"], q["drafted_at"]
            x = reps[c2]["draft"]
            pl = view.logits_at(j)
            teacher[("draft", c2)] = int(recs[c2]["pdm_argmax"])
            teacher[("accept", i)] = bool(recs[i]["accepted"])
            if not recs[i]["accepted"]:
                teacher[("resample", i)] = int(recs[i]["target_token"])
            u_d, u_a, u_r = float(uni[j + 1, U_DRAFT]), float(uni[j + 1, U_ACCEPT]), float(uni[j + 1, U_RESAMPLE])
            if not topk:
                qw, qZ = sampling.softmax_weights(ql, T)
                dec.sample(("draft", c2), qw, u_d)
                pw, pZ = sampling.softmax_weights(pl, T)
                # the accept test u Q(x) < P(x) rests on two single probabilities, so
                # the logit error at x does not average out as in a CDF: the GPU's
                # decision must hold on its own log P(x) - log Q(x) (1e-6), and a
                # differing oracle decision is adopted only if u lies between the
                # oracle's ratio and the GPU's ([YB] 2.1)
                lr_gpu = _log_softmax64(teacher[("plogits", i)], T)[x] - teacher[("qlog", c2)]
                acc_g = u_a < np.exp(lr_gpu)
                if acc_g != bool(recs[i]["accepted"]) and abs(u_a - np.exp(lr_gpu)) > 1e-6:
                    own.mismatch.append((("accept", i), bool(recs[i]["accepted"]), bool(acc_g),
                                         float(abs(u_a - np.exp(lr_gpu)))))
                Px, Qx = float(pw[x]) / pZ, float(qw[x]) / qZ
                shift = abs(np.exp(lr_gpu) - Px / Qx) if Qx > 0 else float("inf")
                dec.lr_err = max(getattr(dec, "lr_err", 0.0), abs(lr_gpu - np.log(Px / Qx)) if Qx > 0 else 0.0)
                if not dec.accept(("accept", i), pw, pZ, qw, qZ, x, u_a, tol=max(STOL[w.dtype], shift)):
                    dec.sample(("resample", i), sampling.residual(pw, pZ, qw, qZ), u_r)
                continue
            Sq = dec.kept_set(("qset", c2), ql, k)
            Sp = dec.kept_set(("pset", i), pl, k)
            eq = eps_of(("qset", c2), ("qval", c2), ql)
            ep = eps_of(("pset", i), ("pval", i), pl)
            # the GPU's own arithmetic on its own logits
            gq_ids, gp_ids = teacher[("qset", c2)], teacher[("pset", i)]
            gqw, gqZ = sampling.softmax_weights(_on_set(w.V, gq_ids, teacher[("qval", c2)]), T, keep=gq_ids)
            gpw, gpZ = sampling.softmax_weights(_on_set(w.V, gp_ids, teacher[("pval", i)]), T, keep=gp_ids)
            own.sample(("draft", c2), gqw, u_d)
            if not own.accept(("accept", i), gpw, gpZ, gqw, gqZ, x, u_a):
                own.sample(("resample", i), sampling.residual(gpw, gpZ, gqw, gqZ), u_r)
            # the oracle's arithmetic on the same sets, within the shift the logit error allows
            qw, qZ = sampling.softmax_weights(ql, T, keep=Sq)
            pw, pZ = sampling.softmax_weights(pl, T, keep=Sp)
            dec.sample(("draft", c2), qw, u_d, tol=max(STOL[w.dtype], sampling.cdf_shift_bound(eq, T)))
            Px, Qx = float(pw[x]) / pZ, float(qw[x]) / qZ
            ok = dec.accept(("accept", i), pw, pZ, qw, qZ, x, u_a,
                            tol=max(STOL[w.dtype], sampling.accept_shift_bound(ep, eq, Px, Qx, u_a, T)))
            if not ok:
                P, Q = pw.astype(np.float64) / pZ, qw.astype(np.float64) / qZ
                dec.sample(("resample", i), sampling.residual(pw, pZ, qw, qZ), u_r,
                           tol=max(STOL[w.dtype], sampling.residual_shift_bound(ep, eq, P, Q, T)))
        if progress:
            progress(f"sampling check: {b0 + len(batch)} of {len(exits)} verifications")
    dec.checked = len(exits)
    dec.own = own
    return dec


def check_floats(run: dict, view: OracleView, reps) -> dict:
    """rel-L2 of the GPU's logits, draft logits, anchors and KV entries at the
    two stopping points against the oracle's; returns the worst of each."""
    w = run["w"]
    worst = {"logits": 0.0, "pdm_logits": 0.0, "anchors": 0.0, "kv": 0.0}
    seen = {k: 0 for k in worst}
    for snap in (run["mid"], run["end"]):
        if "logits" in snap:
            j = reps[snap["exit_index"]]["exit_pos"]
            worst["logits"] = max(worst["logits"], rel_l2(snap["logits"], view.logits_at(j)))
            seen["logits"] += 1
        q = reps[snap["index"]]
        if q["t"] < view.N and view.survived(q):
            worst["pdm_logits"] = max(worst["pdm_logits"], rel_l2(snap["pdm_logits"], view.pdm_logits(q)))
            seen["pdm_logits"] += 1
        t, a = q["t"], q["a"]
        for i, p in enumerate(range(t, t - a, -1)):  # newest first; depth after the step = i + 1
            if p >= view.N or not view.survived(q, upto=p):
                continue
            f = schedule.pattern(i + 1, w.anchors, w.L, w.n, w.split)
            for b in range(f + 1):
                worst["anchors"] = max(worst["anchors"], rel_l2(snap["anchors"][p][b], view.taps[p][b]))
                seen["anchors"] += 1
    kvlen = run["recs"][-1]["kv_len"]
    for l, (K, V) in run["end"]["kv"].items():
        m = min(int(kvlen[l]), view.N)
        worst["kv"] = max(worst["kv"], rel_l2(K[:m], view.tgt.kv[l].K[:m]), rel_l2(V[:m], view.tgt.kv[l].V[:m]))
        seen["kv"] += 1
    worst["seen"] = seen
    return worst
