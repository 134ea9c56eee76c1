"""Closed forms of the SPD schedule (test infrastructure only).

Conventions: positions and layers are 0-indexed; stage k (0..n-1) holds
layers k*L/n .. (k+1)*L/n - 1 under the uniform split, or the next `split[k]`
layers under a non-uniform split; the depth of a token is the number of
stages it has completed (0..n); anchor b means the residual stream after b
layers (b = 0 is the token embedding).

Non-uniform split ([RB] limitations and future work: splits such as
"5+4;9;9;9", whose first rank holds a 5-layer stage and the 4-layer draft
module beside three 9-layer stages, to fit 4- or 8-GPU nodes; [TW] §11 on
balancing stages of a hybrid model).  Reading: `split` lists the layers of
stages 0..n-1 (each >= 1, summing to L); a token at depth k has run the
first split[0] + ... + split[k-1] layers, and every definition below that
the pages state with k*L/n takes that cumulative count instead.
"""
from __future__ import annotations

from typing import List, Optional, Sequence


def stage_sizes(L: int, n: int, split: Optional[Sequence[int]] = None) -> List[int]:
    """Layers per stage: `split` when given, else L/n each ([RB] core method)."""
    if split:
        return [int(x) for x in split]
    return [L // n] * n


def lmax(k: int, L: int, n: int, split: Optional[Sequence[int]] = None) -> int:
    """Deepest layer index a token at depth k has reached: min(L, k*L/n)
    ([RB] core method, bounded incompleteness; [PL] §3.2), or the first k
    stages' layers under a non-uniform split."""
    if split:
        return sum(split[:k])
    return min(L, k * (L // n))


def pattern(k: int, anchors: Sequence[int], L: int, n: int, split: Optional[Sequence[int]] = None) -> int:
    """f(k) = max{i : b_i <= lmax(k)}: the last anchor reachable at depth k.

    The feature of a depth-k token concatenates anchors 0..f(k).  [RB] core
    method; [PL] §3.2 (k = 0 reduces to the embedding alone).
    """
    lm = lmax(k, L, n, split)
    return max(i for i, b in enumerate(anchors) if b <= lm)


def pattern_table(anchors: Sequence[int], L: int, n: int, split: Optional[Sequence[int]] = None) -> List[int]:
    return [pattern(k, anchors, L, n, split) for k in range(n + 1)]


def n_patterns(anchors: Sequence[int], L: int, n: int, split: Optional[Sequence[int]] = None) -> int:
    """Number of distinct fusion projections the depths 0..n use.

    [RB] method step 3: several depths share one fusion pattern when m < n+1;
    [RB] technical novelty: the L=32, n=8 example needs m = 5 projections.
    """
    return len(set(pattern_table(anchors, L, n, split)))


def stage_layers(k: int, L: int, n: int, split: Optional[Sequence[int]] = None) -> range:
    """Layers of stage k: L/n each under the uniform split ([RB] core method),
    the next split[k] layers under a non-uniform one."""
    sizes = stage_sizes(L, n, split)
    start = sum(sizes[:k])
    return range(start, start + sizes[k])


def depth_layout(a: int, pending: bool, n: int) -> List[int]:
    """Depths of the trailing feature rows the draft module sees pre-step.

    Rows are ordered by position.  The just-verified position (if its
    full-depth feature is not cached yet) is at depth n; the a in-flight
    tokens are at depths a-1 .. 0, the newest contributing the embedding
    only.  Steady state (a = n) is the staircase g_n, g_{n-1}, ..., g_0 of
    [RB] method step 2 / [PL] appendix A intro; warm-up (a < n) is the
    shortened staircase of [PL] §A.2 with the prefix at depth n.
    """
    return ([n] if pending else []) + list(range(a - 1, -1, -1))


def post_depth_layout(a: int, n: int) -> List[int]:
    """Depths of the draft module's rows under the post-step schedule.

    After the stage step every token of the pre-step layout is one stage
    deeper: the a tokens in flight at entry sit at depths a .. 1, and when
    a = n the oldest of them has just exited at depth n (its row is the
    full-depth row, committed in the same cycle; no row waits for the next
    cycle).  [PL] §3.3 and the scheduling ablation of [PL] §4 describe the
    post-step features only as "after the pipeline step"; this is that
    reading.
    """
    return list(range(a, 0, -1))


def key_depth(t: int, T: int, fill: int, n: int) -> int:
    """Depth at which position T appears in the feature sequence of step t.

    [PL] §A.3: a query at step t and depth d sees key T at depth
    min(n, d + t - T); keys further back than the fill level are redirected to
    the deepest block.  For the newest query (d = 0) with `fill` tokens in
    flight this is t - T when t - T < fill, else n.  Used as an independent
    formulation that pins `depth_layout` and the state machine's depths.
    """
    assert T <= t
    dist = t - T
    return dist if dist < fill else n


def cycle_count(n: int, G: int, rejects: int) -> int:
    """Cycles needed to emit G tokens (the first from prefill) with R rejects.

    Derived here from the schedule, not printed on the pages: the first exit
    happens at cycle n; every later verification needs one more cycle, and a
    rejection among the first G-2 verifications costs n-1 refill cycles.
    [TW] §8 defines alpha = N/K and the SPD speedup alpha*n from this count.
    """
    return n + (G - 2) + (n - 1) * rejects


def validate_shape(L: int, n: int, Ls: int, anchors: Sequence[int], split: Optional[Sequence[int]] = None) -> None:
    """Constraints the pages fix: n | L ([RB] core method), Ls <= L/n
    ([RB] core method / technical novelty: S = S0 iff Ls <= L/n), anchors
    strictly increasing from 0 and within L ([RB] core method).  A
    non-uniform split lists n stages of >= 1 layers summing to L, and the
    draft module may be as deep as the longest stage (reading: a cycle lasts
    as long as its longest stage; the "5+4;9;9;9" example pairs a 4-layer
    module with 9-layer stages)."""
    if split:
        if len(split) != n or min(split) < 1 or sum(split) != L:
            raise ValueError("a split lists n stages of >= 1 layers summing to L")
        if Ls > max(split):
            raise ValueError("draft module deeper than the longest stage")
    else:
        if L % n:
            raise ValueError("n must divide L")
        if Ls > L // n:
            raise ValueError("draft module deeper than one stage")
    if anchors[0] != 0 or any(b >= c for b, c in zip(anchors, anchors[1:])) or anchors[-1] > L:
        raise ValueError("anchors must increase strictly from 0 and stay <= L")
