"""The benchmark's algorithmic bytes per cycle against an independent count.

A full cycle of the 4B-class n=8 workload streams every target layer once
(32 x 90,439,680 bf16 parameters), the verification head and the draft head
(151936 x 2560 each), all five anchor-fusion matrices (sum (f+1) d^2 for
f = 0..4 = 15 d^2), the Ls = 4 draft layers, and the KV history of every
(token, layer) it attends over -- about 8.31 GB at a context of ~600.  The
count below is written from those shapes, not from bench.py's formula.
"""
import pytest

import bench
import seeded_inputs as si

LAYER_4B = 90_439_680  # 2560 x (20 + 8) x 128 + 2560 x 2560 + 3 x 2560 x 9728


def _rec(t, a, exit_pos, pending):
    return {"t": t, "occupancy": a, "exit_pos": exit_pos, "pending_row": pending}


def test_layer_parameter_count():
    d, Hq, Hkv, hd, F = 2560, 20, 4, 128, 9728
    assert d * (Hq + 2 * Hkv) * hd + Hq * hd * d + 3 * d * F == LAYER_4B


def test_full_cycle_of_4b_n8():
    w = si.workload("4b_n8")
    t, n = 600, 8
    kv_pos = 2 * 4 * 128 * 2                       # k and v of one position, bf16
    per = 4
    kv = sum(per * (t - k + 1) * kv_pos for k in range(n))  # stage k holds position t - k
    heads = 2 * 151936 * 2560 * 2
    fc = 15 * 2560 * 2560 * 2
    draft_layers = 4 * LAYER_4B * 2 + 4 * (t + 1) * kv_pos
    want = 32 * LAYER_4B * 2 + heads + fc + draft_layers + kv
    got = bench.cycle_bytes(w, _rec(t, n, t - n + 1, 1), 2)
    assert got == want
    assert 8.25e9 < got < 8.40e9


def test_warm_up_cycle_counts_only_active_stages_and_present_patterns():
    w = si.workload("4b_n8")
    got = bench.cycle_bytes(w, _rec(600, 1, -1, 0), 2)
    kv_pos = 2 * 4 * 128 * 2
    # one stage (4 layers), no exit head, one fusion pattern (depth 0: the embedding only)
    want = 4 * LAYER_4B * 2 + 4 * 601 * kv_pos + 1 * 2560 * 2560 * 2 + 4 * LAYER_4B * 2 \
        + 151936 * 2560 * 2 + 4 * 601 * kv_pos
    assert got == want


def test_hybrid_linear_layers_move_their_state_instead_of_kv():
    w = si.workload("4b_hybrid_n8")
    t, a = 600, 8
    full = bench.cycle_bytes(si.workload("4b_n8"), _rec(t, a, t - a + 1, 1), 2)
    hyb = bench.cycle_bytes(w, _rec(t, a, t - a + 1, 1), 2)
    kv_pos = 2 * 4 * 128 * 2
    state = 2 * 4 * (128 * 128 + 128) * 4
    delta = 0
    for k in range(a):
        for l in range(4 * k, 4 * k + 4):
            if l % 4 != 3:  # linear layer
                delta += state - (t - k + 1) * kv_pos
    assert hyb - full == delta


def test_post_step_patterns():
    pre_w = si.workload("4b_n8")
    post_w = pre_w.replace(schedule="post")
    # two tokens in flight: pre-step depths 1, 0 use pattern 0 only; post-step
    # depths 2, 1 use patterns 1 (lmax(2) = 8 reaches anchor b = 8) and 0
    pre = bench.cycle_bytes(pre_w, _rec(600, 2, -1, 0), 2)
    post = bench.cycle_bytes(post_w, _rec(600, 2, -1, 0), 2)
    assert post - pre == 2 * 2560 * 2560 * 2
    # full pipeline: post-step depths 8 .. 1 and pre-step depths (8), 7 .. 0 both use all five
    assert bench.cycle_bytes(post_w, _rec(600, 8, 593, 0), 2) == bench.cycle_bytes(pre_w, _rec(600, 8, 593, 1), 2)


def test_non_uniform_split():
    """4b_split_n4 (stages of 5, 9, 9 and 9 layers): active stages stream
    their own layer counts, and the patterns of depths 4 .. 0 are f = 4, 2,
    1, 0, 0 (lmax = 32, 23, 14, 5, 0), so the fusion matrices 0, 1, 2 and 4
    are read: (1 + 2 + 3 + 5) d^2."""
    w = si.workload("4b_split_n4")
    t, n = 600, 4
    sizes = [5, 9, 9, 9]
    kv_pos = 2 * 4 * 128 * 2
    kv = sum(sizes[k] * (t - k + 1) * kv_pos for k in range(n))
    heads = 2 * 151936 * 2560 * 2
    fc = 11 * 2560 * 2560 * 2
    draft_layers = 4 * LAYER_4B * 2 + 4 * (t + 1) * kv_pos
    assert bench.cycle_bytes(w, _rec(t, n, t - n + 1, 1), 2) == 32 * LAYER_4B * 2 + heads + fc + draft_layers + kv
    # warm-up with one token in flight: stage 0's 5 layers, pattern 0 only
    want = 5 * LAYER_4B * 2 + 5 * 601 * kv_pos + 2560 * 2560 * 2 + 4 * LAYER_4B * 2 + 151936 * 2560 * 2 \
        + 4 * 601 * kv_pos
    assert bench.cycle_bytes(w, _rec(600, 1, -1, 0), 2) == want
