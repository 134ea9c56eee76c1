"""The C-ABI library loads and exports every symbol include/spd.h declares;
host-only calls validate configurations (CPU only, no compute calls)."""
import ctypes
import os
import re

import pytest

import seeded_inputs as si
from pipelined_draft_verify_amd import _abi as A
from pipelined_draft_verify_amd.engine import REC_DTYPE, make_config

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spd.h")


def _declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:SPD_API\s+)?(?:const\s+)?\w+\s*\*?\s*(spd_\w+)\s*\(", txt, flags=re.M)))


def test_header_declares_the_boundary():
    names = _declared()
    for n in ("spd_workspace_bytes", "spd_init", "spd_prefill", "spd_cycle", "spd_rollback", "spd_destroy",
              "spd_strerror"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = A.lib()
    missing = [n for n in _declared() if not hasattr(L, n)]
    assert not missing
    assert sorted(n for n, _, _ in A.SIGNATURES) == _declared()


def test_struct_sizes_match_header_layout():
    # spd_cycle_rec: 12 words + 64 KV lengths + the tree fields
    assert ctypes.sizeof(A.spd_cycle_rec) == 4 * (12 + A.SPD_MAX_LAYERS + 3 + 2 * A.SPD_MAX_WIDTH) \
        == REC_DTYPE.itemsize
    assert ctypes.sizeof(A.spd_config) == 4 * (10 + A.SPD_MAX_ANCHORS + 4 + 3 + 3 + A.SPD_MAX_STAGES + 1)
    assert ctypes.sizeof(A.spd_weights) == 8 * (1 + 6 * A.SPD_MAX_LAYERS + 2 + A.SPD_MAX_ANCHORS
                                                + 6 * A.SPD_MAX_PDM_LAYERS + 2)


def test_strerror_and_workspace_sizing_on_host():
    assert A.spd_strerror(0) == "ok"
    assert "state" in A.spd_strerror(A.SPD_ESTATE)
    w = si.workload("4b_n8")
    n = A.spd_workspace_bytes(make_config(w))
    # KV caches (target + draft): (L + Ls) * 2 * Hkv * hd * ctx * 2 bytes, and the
    # draft module's layer matrices in matrix-core tile order (Ls layers, bf16)
    kv = (w.L + w.Ls) * 2 * w.Hkv * w.hd * 1024 * 2
    tiles = w.Ls * ((w.Hq + 2 * w.Hkv) * w.hd * w.d + w.d * w.Hq * w.hd + 3 * w.F * w.d) * 2
    assert kv + tiles < n < (kv + tiles) * 1.5


@pytest.mark.parametrize("field,value", [
    ("n_stages", 3),        # does not divide 32
    ("pdm_layers", 5),      # deeper than one stage (32/8 = 4)
    ("head_dim", 96),
    ("n_kv_heads", 3),      # 20 % 3 != 0
    ("d_model", 2500),      # not a multiple of 256
    ("max_new", 0),
])
def test_invalid_configs_are_rejected(field, value):
    c = make_config(si.workload("4b_n8"))
    setattr(c, field, value)
    with pytest.raises(A.SPDError) as e:
        A.spd_workspace_bytes(c)
    assert e.value.code == A.SPD_EINVAL


def test_anchor_constraints_are_checked():
    c = make_config(si.workload("4b_n8"))
    c.anchors[0] = 1
    with pytest.raises(A.SPDError):
        A.spd_workspace_bytes(c)
    c = make_config(si.workload("4b_n8"))
    c.anchors[2] = c.anchors[1]
    with pytest.raises(A.SPDError):
        A.spd_workspace_bytes(c)
    c = make_config(si.workload("4b_n8"))
    c.anchors[4] = 33
    with pytest.raises(A.SPDError):
        A.spd_workspace_bytes(c)


def test_stage_count_limit():
    """n_stages beyond SPD_MAX_STAGES is rejected even when it divides n_layers."""
    c = make_config(si.workload("4b_n16"))
    assert A.spd_workspace_bytes(c) > 0
    c.n_stages, c.pdm_layers = 32, 1
    with pytest.raises(A.SPDError) as e:
        A.spd_workspace_bytes(c)
    assert e.value.code == A.SPD_EINVAL


def test_vocab_limit():
    """A vocabulary beyond SPD_MAX_VOCAB (the sampler's block-sum capacity) is rejected."""
    c = make_config(si.workload("4b_n8"))
    c.vocab = A.SPD_MAX_VOCAB
    assert A.spd_workspace_bytes(c) > 0
    c.vocab = A.SPD_MAX_VOCAB + 1
    with pytest.raises(A.SPDError) as e:
        A.spd_workspace_bytes(c)
    assert e.value.code == A.SPD_EINVAL


def test_top_k_limits():
    """top_k within [0, min(SPD_MAX_TOPK, vocab)]; a schedule outside SPD_SCHED_* is rejected."""
    c = make_config(si.workload("9b_sample"))
    for k in (0, 1, 50, A.SPD_MAX_TOPK):
        c.top_k = k
        assert A.spd_workspace_bytes(c) > 0
    for k in (-1, A.SPD_MAX_TOPK + 1):
        c.top_k = k
        with pytest.raises(A.SPDError) as e:
            A.spd_workspace_bytes(c)
        assert e.value.code == A.SPD_EINVAL
    c.top_k = 0
    c.schedule = 2
    with pytest.raises(A.SPDError):
        A.spd_workspace_bytes(c)


def test_post_step_needs_two_stages():
    c = make_config(si.workload("4b_n8"))
    c.n_layers, c.n_stages, c.pdm_layers, c.n_anchors = 4, 1, 1, 2
    c.anchors[0], c.anchors[1] = 0, 4
    assert A.spd_workspace_bytes(c) > 0
    c.schedule = A.SPD_SCHED_POST
    with pytest.raises(A.SPDError):
        A.spd_workspace_bytes(c)


def test_attn_period_limits():
    c = make_config(si.workload("4b_n8"))
    for p in (0, 1, 4, 32):
        c.attn_period = p
        assert A.spd_workspace_bytes(c) > 0
    for p in (-1, 33):
        c.attn_period = p
        with pytest.raises(A.SPDError):
            A.spd_workspace_bytes(c)


def test_stage_split_constraints_are_checked():
    w = si.workload("4b_split_n4")
    A.spd_workspace_bytes(make_config(w))              # 5 + 9 + 9 + 9 with a 4-layer draft module
    A.spd_workspace_bytes(make_config(w.replace(Ls=8)))  # as deep as the longest stage
    A.spd_workspace_bytes(make_config(w.replace(n=3, split=(10, 11, 11))))  # n need not divide L
    for kw in [dict(split=(5, 9, 9, 8)),                # sums to 31
               dict(split=(0, 14, 9, 9)),               # an empty stage
               dict(Ls=10),                             # deeper than the longest stage
               dict(n=3, split=(5, 9, 9, 9))]:          # more entries than stages
        with pytest.raises(A.SPDError) as e:
            A.spd_workspace_bytes(make_config(w.replace(**kw)))
        assert e.value.code == A.SPD_EINVAL


def test_static_scratch_state_query_on_host():
    """The allocation-free init's size query: the state is the workspace less
    the scratch, and every named workload's scratch fits the static array."""
    for name in si.WORKLOADS:
        c = make_config(si.workload(name))
        total = A.spd_workspace_bytes(c)
        state = A.spd_init_static_scratch(c)
        assert 0 < state < total
        assert total - state <= A.SPD_STATIC_SCRATCH_MB << 20, name


def test_static_scratch_rejects_oversized_configs():
    c = make_config(si.workload("9b_n8"), max_ctx=32768)
    c.n_stages, c.pdm_layers = 16, 2
    A.spd_workspace_bytes(c)  # a valid configuration ...
    with pytest.raises(A.SPDError) as e:
        A.spd_init_static_scratch(c)  # ... whose scratch exceeds the static array
    assert e.value.code == A.SPD_ESCRATCH


def test_tree_constraints_are_checked():
    """Draft trees are greedy, pre-step, softmax-attention, uniform-stage
    configurations of two or more stages whose draft-module rows
    (2 + (n - 1) W) fit two row tiles; width 0 or 1 is a chain."""
    w = si.workload("4b_tree4_n8")
    assert A.spd_workspace_bytes(make_config(w)) > 0
    for width in (0, 1, 2, 3):
        assert A.spd_workspace_bytes(make_config(w.replace(width=width))) > 0
    # n = 16 at width 2 is exactly 32 rows; width 3 is 47
    assert A.spd_workspace_bytes(make_config(si.workload("4b_n16").replace(width=2))) > 0
    for kw in [dict(width=-1), dict(width=5),                     # outside 0..SPD_MAX_WIDTH
               dict(mode="sample", temperature=1.0),              # greedy only
               dict(schedule="post"),                             # pre-step only
               dict(n=1),                                         # at least two stages
               dict(attn_period=4),                               # softmax attention only
               dict(n=4, split=(5, 9, 9, 9))]:                    # uniform stages only
        with pytest.raises(A.SPDError) as e:
            A.spd_workspace_bytes(make_config(w.replace(**kw)))
        assert e.value.code == A.SPD_EINVAL, kw
        if "width" not in kw:  # the same setting is a valid chain: the tree rule refused it
            assert A.spd_workspace_bytes(make_config(w.replace(width=1, **kw))) > 0, kw
    with pytest.raises(A.SPDError) as e:
        A.spd_workspace_bytes(make_config(si.workload("4b_n16").replace(width=3)))
    assert e.value.code == A.SPD_EINVAL
