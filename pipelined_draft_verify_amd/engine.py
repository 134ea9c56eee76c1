"""SPDEngine: PyTorch-ROCm plumbing around libspd (device memory and streams only).

The engine allocates the workspace and the caller-owned policy arrays with
torch, creates the two default-priority HIP streams, and calls the C ABI.
Every step of the SPD cycle runs in the library's kernels.
"""
from __future__ import annotations

import ctypes
from typing import Dict, List, Optional

import numpy as np

from . import _abi as A

REC_DTYPE = np.dtype([
    ("cycle", "<i4"), ("t", "<i4"), ("occupancy", "<i4"), ("pending_row", "<i4"),
    ("pdm_argmax", "<i4"), ("draft", "<i4"), ("exit_pos", "<i4"), ("target_token", "<i4"),
    ("accepted", "<i4"), ("pdm_len", "<i4"), ("emitted", "<i4"), ("flags", "<u4"),
    ("kv_len", "<i4", (A.SPD_MAX_LAYERS,)),
    ("nodes", "<i4"), ("n_new", "<i4"), ("new_parent", "<i4", (A.SPD_MAX_WIDTH,)),
    ("new_token", "<i4", (A.SPD_MAX_WIDTH,)), ("accepted_rank", "<i4"),
])
assert REC_DTYPE.itemsize == ctypes.sizeof(A.spd_cycle_rec)


def make_config(w, max_ctx: Optional[int] = None) -> A.spd_config:
    c = A.spd_config()
    c.n_layers, c.d_model, c.n_heads, c.n_kv_heads = w.L, w.d, w.Hq, w.Hkv
    c.head_dim, c.d_ffn, c.vocab = w.hd, w.F, w.V
    c.n_stages, c.pdm_layers, c.n_anchors = w.n, w.Ls, len(w.anchors)
    for i, b in enumerate(w.anchors):
        c.anchors[i] = b
    c.dtype = A.SPD_DTYPE_BF16 if w.dtype == "bf16" else A.SPD_DTYPE_F32
    c.max_ctx = max_ctx if max_ctx is not None else w.max_ctx
    c.max_new = w.G
    c.mode = A.SPD_MODE_SAMPLE if w.mode == "sample" else A.SPD_MODE_GREEDY
    c.rms_eps, c.rope_base, c.temperature = w.eps, w.rope_base, w.temperature
    c.schedule = A.SPD_SCHED_POST if getattr(w, "schedule", "pre") == "post" else A.SPD_SCHED_PRE
    c.top_k = getattr(w, "top_k", 0)
    c.attn_period = getattr(w, "attn_period", 0)
    for k, n_k in enumerate(getattr(w, "split", ()) or ()):
        c.stage_layers[k] = n_k
    c.draft_width = getattr(w, "width", 1)
    return c


def make_weights_struct(w, T: Dict[str, "object"]) -> A.spd_weights:
    s = A.spd_weights()
    p = lambda name: T[name].data_ptr()

    def layer(dst, prefix):
        for k in ("attn_norm", "w_qkv", "w_o", "ffn_norm", "w_gu", "w_down"):
            setattr(dst, k, p(prefix + k))
    s.embed = p("embed")
    for i in range(w.L):
        layer(s.layers[i], f"layers.{i}.")
    s.final_norm, s.lm_head = p("final_norm"), p("lm_head")
    for f in range(len(w.anchors)):
        s.fc[f] = p(f"fc.{f}")
    for i in range(w.Ls):
        layer(s.pdm[i], f"pdm_layers.{i}.")
    s.pdm_final_norm, s.pdm_lm_head = p("pdm_final_norm"), p("pdm_lm_head")
    return s


class SPDEngine:
    """One libspd handle on one GPU, with torch-owned workspace and streams."""

    def __init__(self, w, tensors: Dict[str, "object"], device: str = "cuda:0", max_ctx: Optional[int] = None,
                 static_scratch: bool = False):
        """static_scratch: initialise with spd_init_static_scratch -- the
        workspace holds only the persistent state, the per-cycle scratch is
        the library's static device array (shared by every such engine on the
        GPU: their work must not overlap)."""
        import torch

        self.torch = torch
        self.w = w
        self.device = torch.device(device)
        for k, t in tensors.items():
            if t.device != self.device or not t.is_contiguous():
                raise ValueError(f"tensor {k} must be contiguous on {self.device}")
        self.tensors = tensors
        self.cfg = make_config(w, max_ctx)
        self.static_scratch = static_scratch
        self.ws_bytes = (A.spd_init_static_scratch(self.cfg) if static_scratch
                         else A.spd_workspace_bytes(self.cfg))
        self.ws = torch.empty(self.ws_bytes + 256, dtype=torch.uint8, device=self.device)
        base = self.ws.data_ptr()
        self.ws_ptr = (base + 255) // 256 * 256
        self.s_stage = torch.cuda.Stream(device=self.device)
        self.s_pdm = torch.cuda.Stream(device=self.device)
        self.wstruct = make_weights_struct(w, tensors)
        torch.cuda.synchronize(self.device)
        if static_scratch:
            self.h = A.spd_init_static_scratch(self.cfg, self.wstruct, self.ws_ptr, self.ws_bytes,
                                               self.s_stage.cuda_stream, self.s_pdm.cuda_stream)
        else:
            self.h = A.spd_init(self.cfg, self.wstruct, self.ws_ptr, self.ws_bytes,
                                self.s_stage.cuda_stream, self.s_pdm.cuda_stream)
        self.uni = None
        self.ref = None
        self.P = 0
        self.records: List[np.ndarray] = []

    # -- policy / inputs ---------------------------------------------------
    def set_uniforms(self, uni: np.ndarray) -> None:
        t = self.torch.from_numpy(np.ascontiguousarray(uni, dtype=np.float32)).to(self.device)
        self.sync(raise_on_error=False)  # enqueued cycles may still read the old table
        self.uni = t
        A.spd_set_uniforms(self.h, t.data_ptr(), t.shape[0])

    def set_forced(self, ref_tokens, p_accept: float) -> None:
        t = self.torch.tensor(np.asarray(ref_tokens, dtype=np.int32), device=self.device)
        self.sync(raise_on_error=False)  # enqueued cycles may still read the old reference
        self.ref = t
        A.spd_set_draft_policy(self.h, A.SPD_DRAFT_FORCED, float(p_accept), t.data_ptr(), t.numel())

    def set_tree_forced(self, ref_tokens, p_first: float, p_tree: float) -> None:
        t = self.torch.tensor(np.asarray(ref_tokens, dtype=np.int32), device=self.device)
        self.sync(raise_on_error=False)  # enqueued cycles may still read the old reference
        self.ref = t
        A.spd_set_tree_policy(self.h, float(p_first), float(p_tree), t.data_ptr(), t.numel())

    def set_launch_mode(self, graph: bool, serialized: bool = False) -> None:
        mode = A.SPD_LAUNCH_GRAPH if graph else A.SPD_LAUNCH_EAGER
        if serialized:
            mode |= A.SPD_LAUNCH_SERIALIZED
        A.spd_set_launch_mode(self.h, mode)

    def set_natural(self) -> None:
        A.spd_set_draft_policy(self.h, A.SPD_DRAFT_NATURAL, 0.0, 0, 0)

    # -- decoding ----------------------------------------------------------
    def prefill(self, prompt) -> int:
        self.P = len(prompt)
        return A.spd_prefill(self.h, list(prompt))

    def enqueue(self, n: int, log: bool = True):
        """Enqueue n cycles; returns a pinned buffer with their records (valid after sync)."""
        buf = None
        if log:
            buf = self.torch.empty(n * REC_DTYPE.itemsize, dtype=self.torch.uint8, pin_memory=True)
        A.spd_cycle(self.h, n, buf.data_ptr() if buf is not None else None)
        return buf

    @staticmethod
    def records_of(buf) -> np.ndarray:
        return np.frombuffer(buf.numpy().tobytes(), dtype=REC_DTYPE)

    def run(self, batch: int = 64, max_cycles: int = 1 << 20) -> np.ndarray:
        """Cycle until generation is done; returns every executed cycle's record."""
        out = []
        total = 0
        while total < max_cycles:
            buf = self.enqueue(batch)
            st = self.sync()
            recs = self.records_of(buf)
            out.append(recs[(recs["flags"] & A.SPD_FLAG_IDLE) == 0])
            total += batch
            if st.done:
                break
        return np.concatenate(out) if out else np.zeros(0, REC_DTYPE)

    def sync(self, raise_on_error: bool = True) -> A.spd_status:
        return A.spd_sync(self.h, raise_on_error)

    def rollback(self, keep_len: int, token: int) -> None:
        A.spd_rollback(self.h, keep_len, token)

    def generate_ar(self, n: int) -> List[int]:
        return A.spd_generate_ar(self.h, n)

    def tokens(self, first: int, count: int) -> List[int]:
        return A.spd_read_tokens(self.h, first, count)

    # -- debug views ---------------------------------------------------------
    def _read(self, what, index, shape, dtype):
        out = np.empty(shape, dtype=dtype)
        A.spd_debug_read(self.h, what, index, out.ctypes.data, out.nbytes)
        return out

    def anchors(self, pos: int) -> np.ndarray:
        return self._read(A.SPD_DBG_ANCHORS, pos, (len(self.w.anchors), self.w.d), np.float32)

    def hidden(self, pos: int) -> np.ndarray:
        return self._read(A.SPD_DBG_HIDDEN, pos, (self.w.d,), np.float32)

    def logits(self) -> np.ndarray:
        return self._read(A.SPD_DBG_LOGITS, 0, (self.w.V,), np.float32)

    def pdm_logits(self) -> np.ndarray:
        return self._read(A.SPD_DBG_PDM_LOGITS, 0, (self.w.V,), np.float32)

    def kv(self, layer: int, which: str = "k") -> np.ndarray:
        """Layer's key or value cache [max_ctx, Hkv, hd] as float32."""
        w = self.w
        bf = w.dtype == "bf16"
        raw = self._read(A.SPD_DBG_KV_K if which == "k" else A.SPD_DBG_KV_V, layer,
                         (self.cfg.max_ctx, w.Hkv, w.hd), np.uint16 if bf else np.float32)
        if bf:
            return (raw.astype(np.uint32) << 16).view(np.float32)
        return raw

    # -- timing ------------------------------------------------------------
    def timing(self, enable: bool) -> None:
        A.spd_timing_enable(self.h, enable)

    def timing_read(self, cap: int = 1 << 16):
        return A.spd_timing_read(self.h, cap)

    def close(self) -> None:
        if getattr(self, "h", None):
            A.spd_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
