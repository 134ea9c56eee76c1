"""ctypes mirror of include/spd.h and same-named thin wrappers (marshalling only).

Every compute step runs in libspd's HIP kernels; this module only converts
Python values to the C types of the ABI.  Loading fails loudly when the
library has not been built: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, Structure, c_double, c_float, c_int32, c_size_t, c_uint32, c_void_p

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libspd.so")

SPD_MAX_LAYERS = 64
SPD_MAX_PDM_LAYERS = 8
SPD_MAX_ANCHORS = 8
SPD_MAX_STAGES = 16
SPD_MAX_VOCAB = 1 << 20
SPD_MAX_TOPK = 64
SPD_MAX_WIDTH = 4

SPD_OK, SPD_EINVAL, SPD_ESTATE, SPD_ECTX, SPD_EHIP, SPD_EDEVICE, SPD_ESCRATCH = 0, -1, -2, -3, -4, -5, -6
SPD_STATIC_SCRATCH_MB = 64
SPD_DTYPE_F32, SPD_DTYPE_BF16 = 0, 1
SPD_MODE_GREEDY, SPD_MODE_SAMPLE = 0, 1
SPD_SCHED_PRE, SPD_SCHED_POST = 0, 1
SPD_DRAFT_NATURAL, SPD_DRAFT_FORCED = 0, 1
SPD_U_COUNT = 5
SPD_FLAG_KVLEN, SPD_FLAG_OCCUPANCY, SPD_FLAG_CTX, SPD_FLAG_IDLE, SPD_FLAG_NODRAFT, SPD_FLAG_BADTOKEN = 1, 2, 4, 8, 16, 32
SPD_DBG_ANCHORS, SPD_DBG_HIDDEN, SPD_DBG_LOGITS, SPD_DBG_PDM_LOGITS, SPD_DBG_KV_K, SPD_DBG_KV_V = range(6)


class spd_config(Structure):
    _fields_ = [
        ("n_layers", c_int32), ("d_model", c_int32), ("n_heads", c_int32), ("n_kv_heads", c_int32),
        ("head_dim", c_int32), ("d_ffn", c_int32), ("vocab", c_int32),
        ("n_stages", c_int32), ("pdm_layers", c_int32), ("n_anchors", c_int32),
        ("anchors", c_int32 * SPD_MAX_ANCHORS),
        ("dtype", c_int32), ("max_ctx", c_int32), ("max_new", c_int32), ("mode", c_int32),
        ("rms_eps", c_float), ("rope_base", c_float), ("temperature", c_float),
        ("schedule", c_int32), ("attn_period", c_int32), ("top_k", c_int32),
        ("stage_layers", c_int32 * SPD_MAX_STAGES),
        ("draft_width", c_int32),
    ]


class spd_layer_weights(Structure):
    _fields_ = [(k, c_void_p) for k in ("attn_norm", "w_qkv", "w_o", "ffn_norm", "w_gu", "w_down")]


class spd_weights(Structure):
    _fields_ = [
        ("embed", c_void_p),
        ("layers", spd_layer_weights * SPD_MAX_LAYERS),
        ("final_norm", c_void_p), ("lm_head", c_void_p),
        ("fc", c_void_p * SPD_MAX_ANCHORS),
        ("pdm", spd_layer_weights * SPD_MAX_PDM_LAYERS),
        ("pdm_final_norm", c_void_p), ("pdm_lm_head", c_void_p),
    ]


class spd_cycle_rec(Structure):
    _fields_ = [
        ("cycle", c_int32), ("t", c_int32), ("occupancy", c_int32), ("pending_row", c_int32),
        ("pdm_argmax", c_int32), ("draft", c_int32), ("exit_pos", c_int32), ("target_token", c_int32),
        ("accepted", c_int32), ("pdm_len", c_int32), ("emitted", c_int32), ("flags", c_uint32),
        ("kv_len", c_int32 * SPD_MAX_LAYERS),
        ("nodes", c_int32), ("n_new", c_int32), ("new_parent", c_int32 * SPD_MAX_WIDTH),
        ("new_token", c_int32 * SPD_MAX_WIDTH), ("accepted_rank", c_int32),
    ]


class spd_status(Structure):
    _fields_ = [
        ("cycles", c_int32), ("emitted", c_int32), ("done", c_int32), ("t", c_int32),
        ("occupancy", c_int32), ("pdm_len", c_int32), ("flags", c_uint32), ("hip_error", c_int32),
    ]


# (name, restype, argtypes) of every exported entry point, in header order
SIGNATURES = [
    ("spd_workspace_bytes", c_int32, [POINTER(spd_config), POINTER(c_size_t)]),
    ("spd_init", c_int32, [POINTER(spd_config), POINTER(spd_weights), c_void_p, c_size_t, c_void_p, c_void_p,
                           POINTER(c_void_p)]),
    ("spd_init_static_scratch", c_int32, [POINTER(spd_config), POINTER(spd_weights), c_void_p, POINTER(c_size_t),
                                          c_void_p, c_void_p, POINTER(c_void_p)]),
    ("spd_set_draft_policy", c_int32, [c_void_p, c_int32, c_float, c_void_p, c_int32]),
    ("spd_set_tree_policy", c_int32, [c_void_p, c_float, c_float, c_void_p, c_int32]),
    ("spd_set_launch_mode", c_int32, [c_void_p, c_int32]),
    ("spd_set_uniforms", c_int32, [c_void_p, c_void_p, c_int32]),
    ("spd_prefill", c_int32, [c_void_p, POINTER(c_int32), c_int32, POINTER(c_int32)]),
    ("spd_cycle", c_int32, [c_void_p, c_int32, c_void_p]),
    ("spd_rollback", c_int32, [c_void_p, c_int32, c_int32]),
    ("spd_generate_ar", c_int32, [c_void_p, c_int32, POINTER(c_int32)]),
    ("spd_sync", c_int32, [c_void_p, POINTER(spd_status)]),
    ("spd_read_tokens", c_int32, [c_void_p, c_int32, c_int32, POINTER(c_int32)]),
    ("spd_debug_read", c_int32, [c_void_p, c_int32, c_int32, c_void_p, c_size_t]),
    ("spd_timing_enable", c_int32, [c_void_p, c_int32]),
    ("spd_timing_read", c_int32, [c_void_p, c_int32, POINTER(c_float), POINTER(c_double), POINTER(c_int32)]),
    ("spd_destroy", c_int32, [c_void_p]),
    ("spd_strerror", ctypes.c_char_p, [c_int32]),
]

_LIB = None


class SPDError(RuntimeError):
    def __init__(self, fn, code):
        msg = lib().spd_strerror(code).decode() if _LIB is not None else str(code)
        super().__init__(f"{fn} failed: {code} ({msg})")
        self.code = code


def lib():
    """Load libspd.so (built in-tree); raise if it is missing."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "(python -c 'import __graft_entry__ as g; g.build()')")
        try:
            import torch  # noqa: F401  (binds the process to torch's HIP runtime first)
        except Exception:
            pass
        L = ctypes.CDLL(LIB_PATH)
        for name, res, args in SIGNATURES:
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _LIB = L
    return _LIB


def check(fn, code):
    if code != SPD_OK:
        raise SPDError(fn, code)
    return code


# Same-named wrappers ---------------------------------------------------------
def spd_workspace_bytes(cfg: spd_config) -> int:
    n = c_size_t(0)
    check("spd_workspace_bytes", lib().spd_workspace_bytes(ctypes.byref(cfg), ctypes.byref(n)))
    return n.value


def spd_init(cfg, weights, workspace_ptr, ws_bytes, stage_stream, pdm_stream):
    h = c_void_p(0)
    check("spd_init", lib().spd_init(ctypes.byref(cfg), ctypes.byref(weights), c_void_p(workspace_ptr),
                                      c_size_t(ws_bytes), c_void_p(stage_stream), c_void_p(pdm_stream),
                                      ctypes.byref(h)))
    return h


def spd_init_static_scratch(cfg, weights=None, state_ptr=None, state_bytes=0, stage_stream=None, pdm_stream=None):
    """With state_ptr None: the size query, returns the state bytes.  Else
    returns the handle."""
    n = c_size_t(state_bytes)
    if state_ptr is None:
        check("spd_init_static_scratch", lib().spd_init_static_scratch(ctypes.byref(cfg), None, None,
                                                                        ctypes.byref(n), None, None, None))
        return n.value
    h = c_void_p(0)
    check("spd_init_static_scratch", lib().spd_init_static_scratch(
        ctypes.byref(cfg), ctypes.byref(weights), c_void_p(state_ptr), ctypes.byref(n), c_void_p(stage_stream),
        c_void_p(pdm_stream), ctypes.byref(h)))
    return h


def spd_set_draft_policy(h, policy, p_accept, ref_ptr, ref_len):
    return check("spd_set_draft_policy", lib().spd_set_draft_policy(h, policy, p_accept, c_void_p(ref_ptr), ref_len))


def spd_set_tree_policy(h, p_first, p_tree, ref_ptr, ref_len):
    return check("spd_set_tree_policy", lib().spd_set_tree_policy(h, p_first, p_tree, c_void_p(ref_ptr), ref_len))


SPD_LAUNCH_EAGER, SPD_LAUNCH_GRAPH, SPD_LAUNCH_SERIALIZED = 0, 1, 2


def spd_set_launch_mode(h, mode):
    return check("spd_set_launch_mode", lib().spd_set_launch_mode(h, mode))


def spd_set_uniforms(h, uni_ptr, n_positions):
    return check("spd_set_uniforms", lib().spd_set_uniforms(h, c_void_p(uni_ptr), n_positions))


def spd_prefill(h, prompt) -> int:
    arr = (c_int32 * len(prompt))(*[int(x) for x in prompt])
    first = c_int32(-1)
    check("spd_prefill", lib().spd_prefill(h, arr, len(prompt), ctypes.byref(first)))
    return first.value


def spd_cycle(h, n_cycles, log_ptr=None):
    return check("spd_cycle", lib().spd_cycle(h, n_cycles, c_void_p(log_ptr) if log_ptr else None))


def spd_rollback(h, keep_len, token):
    return check("spd_rollback", lib().spd_rollback(h, keep_len, token))


def spd_generate_ar(h, n_tokens):
    out = (c_int32 * max(1, n_tokens))()
    check("spd_generate_ar", lib().spd_generate_ar(h, n_tokens, out))
    return list(out)[:n_tokens]


def spd_sync(h, raise_on_error=True) -> spd_status:
    st = spd_status()
    code = lib().spd_sync(h, ctypes.byref(st))
    if raise_on_error:
        check("spd_sync", code)
    return st


def spd_read_tokens(h, first, count):
    out = (c_int32 * max(1, count))()
    check("spd_read_tokens", lib().spd_read_tokens(h, first, count, out))
    return list(out)[:count]


def spd_debug_read(h, what, index, out_ptr, nbytes):
    return check("spd_debug_read", lib().spd_debug_read(h, what, index, c_void_p(out_ptr), c_size_t(nbytes)))


def spd_timing_enable(h, enable):
    return check("spd_timing_enable", lib().spd_timing_enable(h, 1 if enable else 0))


def spd_timing_read(h, cap):
    buf = (c_float * max(3, 3 * cap))()
    gu = c_double(0)
    ngu = c_int32(0)
    n = lib().spd_timing_read(h, cap, buf, ctypes.byref(gu), ctypes.byref(ngu))
    if n < 0:
        raise SPDError("spd_timing_read", n)
    cyc = [(buf[3 * i], buf[3 * i + 1], buf[3 * i + 2]) for i in range(min(n, cap))]
    return n, cyc, gu.value, ngu.value


def spd_destroy(h):
    return check("spd_destroy", lib().spd_destroy(h))


def spd_strerror(code):
    return lib().spd_strerror(code).decode()
