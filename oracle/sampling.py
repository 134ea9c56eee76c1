"""Temperature sampling and rejection-sampling verification (test infrastructure only).

[YB] §2.1: a draft x drawn from Q is accepted with probability
min(1, P(x)/Q(x)); otherwise the token is redrawn from the adjusted
distribution normalize(max(0, P - Q)).  [YB] §2.2: the emitted token is then
distributed exactly as P.  [TW] §6 / [PL] §3.4: SPD applies this rule at the
streaming verification of each position.

Precision (the decisions are taken the same way on both sides): weights
w_v = exp(l_v/T - max) in float32; normalisers, CDFs and the acceptance
comparison in float64; inverse CDF = smallest id i whose ascending-id
cumulative weight exceeds u * (total weight).

Top-k ([RB] reproducibility assessment: the evaluation decodes with top-k 50,
top-p 1.0): only the k largest logits keep their weight, the others weigh 0;
equal logits rank by the lower id; the selection is on the logits as given
(before the temperature).  Applying the same truncation to P and Q keeps the
rejection rule exact for the truncated target law.  Top-p 1.0 truncates
nothing.
"""
from __future__ import annotations

import numpy as np


def top_k_ids(logits: np.ndarray, k: int) -> np.ndarray:
    """Ids of the k largest logits in ascending id order; equal logits rank
    by the lower id (a stable sort on the negated value)."""
    l = np.asarray(logits, np.float32)
    order = np.lexsort((np.arange(len(l)), -l))
    return np.sort(order[:k])


def top_k_set_gap(logits: np.ndarray, ids) -> float:
    """How far the id set `ids` is from being a top-|ids| set of `logits`:
    the largest logit left out minus the smallest logit kept (0 when no
    excluded id beats a kept one).  The set is decided by logit comparisons
    like an argmax, so a second implementation whose logits differ by rounding
    may keep another set; it is a valid top-k choice when this gap is within
    the argmax tolerance (for k = 1 this is the argmax near-tie rule)."""
    l = np.asarray(logits, np.float32)
    ids = np.asarray(ids, np.int64)
    if len(ids) == 0 or len(ids) >= len(l):
        return 0.0
    out = np.ones(len(l), bool)
    out[ids] = False
    return float(max(0.0, float(l[out].max()) - float(l[ids].min())))


def softmax_weights(logits: np.ndarray, temperature: float = 1.0, top_k: int = 0, keep=None):
    """(w float32, Z float64): unnormalised softmax weights and their sum;
    with top_k > 0 only the top-k ids keep their weight (or, when `keep` is
    given, the ids it lists: a kept set decided elsewhere)."""
    l = logits.astype(np.float32)
    if temperature != 1.0:
        l = l / np.float32(temperature)
    w = np.exp(l - l.max()).astype(np.float32)
    if keep is not None or 0 < top_k < len(w):
        mask = np.zeros(len(w), bool)
        mask[top_k_ids(logits, top_k) if keep is None else np.asarray(keep, np.int64)] = True
        w = np.where(mask, w, np.float32(0)).astype(np.float32)
    return w, float(np.sum(w.astype(np.float64)))


def inverse_cdf(weights: np.ndarray, u: float):
    """Smallest i with cumsum(weights)[i] > u * sum(weights) (float64 cumsum).

    Returns (index, gap) where gap is the distance of the threshold from the
    nearest boundary of the chosen interval, relative to the total (used to
    judge whether another implementation may legitimately differ).
    """
    c = np.cumsum(weights.astype(np.float64))
    total = c[-1]
    thr = np.float64(u) * total
    i = int(np.searchsorted(c, thr, side="right"))
    if i >= len(c):
        i = int(np.flatnonzero(weights > 0)[-1])
    lo = c[i - 1] if i > 0 else 0.0
    gap = min(thr - lo, c[i] - thr) / total if total > 0 else 0.0
    return i, float(gap)


def accept_test(p_w, p_Z, q_w, q_Z, x: int, u: float):
    """Accept draft x iff u * Q(x) < P(x)  (i.e. u < min(1, P/Q)).

    Returns (accepted, gap): gap = |u*Q(x) - P(x)| / Q(x).
    """
    Px = np.float64(p_w[x]) / p_Z
    Qx = np.float64(q_w[x]) / q_Z
    lhs = np.float64(u) * Qx
    return bool(lhs < Px), float(abs(lhs - Px) / Qx) if Qx > 0 else float("inf")


def residual(p_w, p_Z, q_w, q_Z) -> np.ndarray:
    """max(0, P - Q) (float64, unnormalised: inverse_cdf normalises)."""
    P = p_w.astype(np.float64) / p_Z
    Q = q_w.astype(np.float64) / q_Z
    return np.maximum(0.0, P - Q)


def emit_distribution(P: np.ndarray, Q: np.ndarray) -> np.ndarray:
    """Exact law of the token the rule emits when x ~ Q (for enumeration pins).

    Pr[emit v] = Q(v) min(1, P(v)/Q(v)) + (1 - sum_x min(P(x), Q(x))) r(v),
    with r = normalize(max(0, P - Q)).  [YB] §2.2 states that this equals P.
    """
    P = P.astype(np.float64)
    Q = Q.astype(np.float64)
    acc = np.where(Q > 0, Q * np.minimum(1.0, np.divide(P, Q, out=np.zeros_like(P), where=Q > 0)), 0.0)
    rej_mass = 1.0 - np.minimum(P, Q).sum()
    r = np.maximum(0.0, P - Q)
    r = r / r.sum() if r.sum() > 0 else np.zeros_like(P)
    return acc + rej_mass * r


def cdf_shift_bound(eps: float, temperature: float = 1.0) -> float:
    """Largest move of any point of a softmax CDF (as a fraction of the mass)
    when every logit moves by at most eps: the mass below a boundary is
    A / (A + B) with A, B scaled by at most exp(+-eps/T), so it moves by at
    most tanh(eps / (2T))."""
    return float(np.tanh(eps / (2.0 * temperature)))


def accept_shift_bound(eps_p: float, eps_q: float, Px: float, Qx: float, u: float, temperature: float = 1.0) -> float:
    """Largest move of the accept-test gap |u Q(x) - P(x)| / Q(x) when P's and
    Q's logits move by at most eps_p, eps_q: each probability moves by a factor
    within exp(+-2 eps / T)."""
    rp = float(np.expm1(2.0 * eps_p / temperature))
    rq = float(np.expm1(2.0 * eps_q / temperature))
    return u * rq + (Px / Qx) * rp if Qx > 0 else float("inf")


def residual_shift_bound(eps_p: float, eps_q: float, P: np.ndarray, Q: np.ndarray, temperature: float = 1.0) -> float:
    """Largest move of a point of the residual max(0, P - Q)'s CDF (fraction of
    its mass): each residual weight moves by at most |dP_v| + |dQ_v| <=
    P_v rp + Q_v rq, so the mass below a boundary and the total move by at
    most D = sum_v (P_v rp + Q_v rq) over the support, and the fraction by at
    most 2 D / (total - D)."""
    rp = float(np.expm1(2.0 * eps_p / temperature))
    rq = float(np.expm1(2.0 * eps_q / temperature))
    r = np.maximum(0.0, P - Q)
    tot = float(r.sum())
    D = float(np.sum((P * rp + Q * rq)[(P > 0) | (Q > 0)]))
    return 2.0 * D / (tot - D) if tot > D else float("inf")
