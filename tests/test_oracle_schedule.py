"""Pins of the oracle's schedule closed forms against the pages' worked examples
and an independent formulation of the depth layout (CPU only)."""
import json
import os

import pytest

from oracle import schedule as S

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "paper_worked_examples.json")))


def test_projection_count_of_worked_example():
    g = GOLD["n_projections"]
    assert S.n_patterns(g["anchors"], g["L"], g["n"]) == g["value"]


def test_k0_reduces_to_embedding_and_full_depth_uses_all_anchors():
    g = GOLD["anchor_example"]
    for n in (2, 4, 8, 16, 32):
        tab = S.pattern_table(g["anchors"], g["L"], n)
        assert tab[0] == GOLD["k0_is_embedding"]["pattern"]
        assert tab[n] == len(g["anchors"]) - 1


def test_anchor_31_is_reached_only_at_full_depth():
    # b=31 lies inside the last stage (layers 28..31 at n=8): a token that has
    # finished 7 stages (28 layers) cannot use it yet.
    g = GOLD["anchor_example"]
    tab = S.pattern_table(g["anchors"], g["L"], 8)
    assert tab[7] == 3 and tab[8] == 4


def test_patterns_monotone_and_shared_when_fewer_anchors_than_depths():
    g = GOLD["anchor_example"]
    for n in (4, 8, 16):
        tab = S.pattern_table(g["anchors"], g["L"], n)
        assert all(a <= b for a, b in zip(tab, tab[1:]))
        # m < n+1 forces at least two depths to share a fusion pattern
        if len(g["anchors"]) < n + 1:
            assert len(set(tab)) < n + 1
    # the anchor chosen is always already computed at that depth
    for n in (4, 8, 16):
        for k in range(n + 1):
            f = S.pattern(k, g["anchors"], g["L"], n)
            assert g["anchors"][f] <= k * g["L"] // n


def test_stage_partition_of_worked_example():
    g = GOLD["stage_partition"]
    sizes = [len(S.stage_layers(k, g["L"], g["n"])) for k in range(g["n"])]
    assert sizes == [g["layers_per_stage"]] * g["n"]
    covered = [l for k in range(g["n"]) for l in S.stage_layers(k, g["L"], g["n"])]
    assert covered == list(range(g["L"]))
    S.validate_shape(g["L"], g["n"], g["max_pdm_layers"], GOLD["anchor_example"]["anchors"])
    with pytest.raises(ValueError):
        S.validate_shape(g["L"], g["n"], g["max_pdm_layers"] + 1, GOLD["anchor_example"]["anchors"])
    with pytest.raises(ValueError):
        S.validate_shape(30, 8, 1, [0, 8])
    with pytest.raises(ValueError):
        S.validate_shape(32, 8, 1, [1, 8])


def test_n4_depth_picture():
    g = GOLD["n4_depth_picture"]
    lay = S.depth_layout(g["n"], False, g["n"])
    assert list(reversed(lay)) == g["in_flight_depths_newest_to_oldest"]


@pytest.mark.parametrize("n", [1, 2, 3, 4, 8, 16])
def test_depth_layout_matches_key_depth_rule(n):
    # Independent formulation: the per-key routing rule of the structural mask
    # gives, for the newest query at step t, the depth of every earlier key.
    for a in range(1, n + 1):
        for pending in (False, True):
            lay = S.depth_layout(a, pending, n)
            t = 100
            start = t - len(lay) + 1
            via_rule = [S.key_depth(t, T, a, n) for T in range(start, t + 1)]
            assert lay == via_rule
            # everything older than the trailing rows sits at full depth
            assert S.key_depth(t, start - 1, a, n) == n


def test_lmax_is_capped_by_L():
    assert S.lmax(8, 32, 8) == 32
    assert S.lmax(3, 32, 8) == 12
    assert S.lmax(0, 32, 8) == 0


def test_cycle_count_small_cases():
    # all accepted: one cycle per verification after an n-cycle fill
    assert S.cycle_count(8, 2, 0) == 8
    assert S.cycle_count(4, 10, 0) == 12
    # every verification rejected: n cycles per token (autoregressive pace)
    n, G = 4, 64
    assert S.cycle_count(n, G, G - 2) == n * (G - 1)
