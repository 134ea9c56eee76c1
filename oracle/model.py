"""Target decoder, draft module (PDM) and multi-depth features (test infrastructure only)."""
from __future__ import annotations

from typing import List, Optional, Sequence

import numpy as np

from .layers import (F32, apply_rope, attention, bf16_round, elu_plus_one, linear_attention, rmsnorm,
                     rope_cos_sin, rope_tables, silu)
from .schedule import pattern, stage_layers


class KVCache:
    """Per-layer key/value store with a length word.

    Entries are kept in the model's storage precision (bf16-rounded for bf16
    models).  `length` is the number of valid positions; truncation is a
    write of the length alone, as in the rollback of [RB] method step 5.
    """

    def __init__(self, max_ctx: int, Hkv: int, hd: int, bf16: bool):
        self.K = np.zeros((max_ctx, Hkv, hd), dtype=F32)
        self.V = np.zeros((max_ctx, Hkv, hd), dtype=F32)
        self.length = 0
        self.bf16 = bf16

    def write(self, pos: int, k: np.ndarray, v: np.ndarray) -> None:
        if self.bf16:
            k, v = bf16_round(k), bf16_round(v)
        self.K[pos] = k
        self.V[pos] = v


def _qkv(lw, u, Hq, Hkv, hd):
    qkv = lw["w_qkv"] @ u
    q = qkv[: Hq * hd].reshape(Hq, hd)
    k = qkv[Hq * hd: (Hq + Hkv) * hd].reshape(Hkv, hd)
    v = qkv[(Hq + Hkv) * hd:].reshape(Hkv, hd)
    return q, k, v


def _ffn(lw, h, F, eps):
    u2 = rmsnorm(h, lw["ffn_norm"], eps)
    gu = lw["w_gu"] @ u2
    return h + lw["w_down"] @ (silu(gu[:F]) * gu[F:])


class _Shape:
    def __init__(self, w):
        self.L, self.d, self.Hq, self.Hkv, self.hd = w.L, w.d, w.Hq, w.Hkv, w.hd
        self.F, self.V, self.n, self.Ls = w.F, w.V, w.n, w.Ls
        self.anchors = list(w.anchors)
        self.eps, self.base = w.eps, w.rope_base
        self.bf16 = w.dtype == "bf16"
        self.max_ctx = w.max_ctx
        self.attn_period = getattr(w, "attn_period", 0)
        self.split = tuple(getattr(w, "split", ()) or ())

    def linear(self, layer: int) -> bool:
        """Hybrid target ([RB] limitations, [TW] §11: each block of 4
        layers holds 1 standard and 3 linear-attention layers).  Reading: with
        period P, layer l uses full softmax attention iff l % P == P - 1 (the
        last of each block), linear attention otherwise; P = 0: all full."""
        P = self.attn_period
        return P > 0 and layer % P != P - 1


def layer_step(s: _Shape, lw, h: np.ndarray, pos: int, kv: KVCache, check_len: bool = True,
               linear: bool = False):
    """One decoder layer for one token at position `pos` (pre-norm, GQA, SwiGLU).

    Appends the token's k, v at index pos (asserting the cache holds exactly
    positions 0..pos-1 when `check_len`) and attends over 0..pos (softmax
    attention, or linear attention for a hybrid target's linear layers).
    """
    u = rmsnorm(h, lw["attn_norm"], s.eps)
    q, k, v = _qkv(lw, u, s.Hq, s.Hkv, s.hd)
    c, sn = rope_cos_sin(pos, s.hd, s.base)
    q, k = apply_rope(q, c, sn), apply_rope(k, c, sn)
    if check_len:
        assert kv.length == pos, f"KV length {kv.length} != position {pos}"
    kv.write(pos, k, v)
    kv.length = pos + 1
    o = (linear_attention if linear else attention)(q, kv.K[: pos + 1], kv.V[: pos + 1])
    h = h + lw["w_o"] @ o.reshape(-1)
    return _ffn(lw, h, s.F, s.eps)


def layer_rows(s: _Shape, lw, X: np.ndarray, pos0: int, kv: KVCache, linear: bool = False) -> np.ndarray:
    """One decoder layer over M consecutive positions pos0..pos0+M-1 (causal).

    Row i attends to cached positions 0..pos0-1 and to rows 0..i.  The rows'
    k, v are written at positions pos0.. of `kv`; whether they stay valid is
    the caller's decision (the length word is not touched).
    """
    M = X.shape[0]
    Q = []
    for i in range(M):
        u = rmsnorm(X[i], lw["attn_norm"], s.eps)
        q, k, v = _qkv(lw, u, s.Hq, s.Hkv, s.hd)
        c, sn = rope_cos_sin(pos0 + i, s.hd, s.base)
        Q.append(apply_rope(q, c, sn))
        kv.write(pos0 + i, apply_rope(k, c, sn), v)
    out = np.empty_like(X)
    for i in range(M):
        p = pos0 + i
        o = (linear_attention if linear else attention)(Q[i], kv.K[: p + 1], kv.V[: p + 1])
        h = X[i] + lw["w_o"] @ o.reshape(-1)
        out[i] = _ffn(lw, h, s.F, s.eps)
    return out


def layer_matrix(s: _Shape, lw, X: np.ndarray, pos0: int, kv: KVCache, linear: bool = False) -> np.ndarray:
    """`layer_rows` written with matrix products over all M rows at once.

    The same definition (row i attends to cached positions and rows <= i,
    masked scores are -inf before the softmax); only the order of
    floating-point operations differs.  Used for long sequences, where the
    row-at-a-time form is too slow; the softmax and SiLU of the big score and
    gate matrices use torch's (multi-threaded) CPU functions as library steps.
    Pinned against `layer_rows` in the CPU tests.
    """
    import torch

    M = X.shape[0]
    Hq, Hkv, hd = s.Hq, s.Hkv, s.hd
    U = np.stack([rmsnorm(X[i], lw["attn_norm"], s.eps) for i in range(M)])
    QKV = U @ lw["w_qkv"].T
    Q = QKV[:, : Hq * hd].reshape(M, Hq, hd)
    Kn = QKV[:, Hq * hd:(Hq + Hkv) * hd].reshape(M, Hkv, hd)
    Vn = QKV[:, (Hq + Hkv) * hd:].reshape(M, Hkv, hd)
    cos, sin = rope_tables(np.arange(pos0, pos0 + M), hd, s.base)
    cos, sin = cos[:, None, :], sin[:, None, :]
    Q = apply_rope(Q, cos, sin)
    Kr = apply_rope(Kn, cos, sin)
    for i in range(M):
        kv.write(pos0 + i, Kr[i], Vn[i])
    T = pos0 + M
    grp = Hq // Hkv
    scale = F32(1.0 / np.sqrt(hd))
    mask = torch.from_numpy(np.arange(T)[None, :] > (pos0 + np.arange(M))[:, None])
    O = np.empty((M, Hq, hd), dtype=F32)
    for h in range(Hq):
        k_ = torch.from_numpy(np.ascontiguousarray(kv.K[:T, h // grp, :]))
        v_ = torch.from_numpy(np.ascontiguousarray(kv.V[:T, h // grp, :]))
        if linear:
            # linear attention: weights phi(q).phi(k), masked to 0, normalised by their sum
            Wt = (torch.from_numpy(np.ascontiguousarray(elu_plus_one(Q[:, h, :])))
                  @ torch.from_numpy(np.ascontiguousarray(elu_plus_one(kv.K[:T, h // grp, :]))).T)
            Wt.masked_fill_(mask, 0.0)
            O[:, h, :] = ((Wt @ v_) / Wt.sum(dim=1, keepdim=True)).numpy()
            continue
        S = (torch.from_numpy(np.ascontiguousarray(Q[:, h, :])) @ k_.T) * float(scale)
        S.masked_fill_(mask, float("-inf"))
        O[:, h, :] = (torch.softmax(S, dim=1) @ v_).numpy()
    H = X + O.reshape(M, Hq * hd) @ lw["w_o"].T
    U2 = np.stack([rmsnorm(H[i], lw["ffn_norm"], s.eps) for i in range(M)])
    GU = torch.from_numpy(np.ascontiguousarray(U2 @ lw["w_gu"].T))
    act = (torch.nn.functional.silu(GU[:, : s.F]) * GU[:, s.F:]).numpy()
    return (H + act @ lw["w_down"].T).astype(F32)


class Target:
    """The L-layer target decoder with per-layer KV caches and anchor taps."""

    def __init__(self, w, W):
        self.s = _Shape(w)
        self.W = W
        self.kv = [KVCache(self.s.max_ctx, self.s.Hkv, self.s.hd, self.s.bf16)
                   for _ in range(self.s.L)]
        # anchor index of each layer boundary b (residual after b layers)
        self.anchor_at = {b: i for i, b in enumerate(self.s.anchors)}

    def embed(self, tok: int) -> np.ndarray:
        return self.W["embed"][tok].astype(F32).copy()

    def run_layers(self, h: np.ndarray, pos: int, layers: Sequence[int],
                   taps: Optional[List] = None) -> np.ndarray:
        """Run `layers` for one token; record anchors h^(b) into `taps`."""
        for l in layers:
            h = layer_step(self.s, self.W["layers"][l], h, pos, self.kv[l], linear=self.s.linear(l))
            if taps is not None and (l + 1) in self.anchor_at:
                taps[self.anchor_at[l + 1]] = h.copy()
        return h

    def run_stage(self, h, pos, k, taps=None):
        return self.run_layers(h, pos, stage_layers(k, self.s.L, self.s.n, self.s.split), taps)

    def logits(self, h: np.ndarray) -> np.ndarray:
        """Full-depth logits W_lm * rmsnorm(h^(L)) (float32)."""
        return self.W["lm_head"] @ rmsnorm(h, self.W["final_norm"], self.s.eps)

    def logits_rows(self, H: np.ndarray) -> np.ndarray:
        """`logits` of every row of H [M, d] with one matrix product: [M, V]."""
        U = np.stack([rmsnorm(h, self.W["final_norm"], self.s.eps) for h in H])
        return (U @ self.W["lm_head"].T).astype(F32)

    def forward_token(self, tok: int, pos: int):
        """Whole-model pass for one token: (final hidden, anchors)."""
        taps = [None] * len(self.s.anchors)
        h = self.embed(tok)
        taps[0] = h.copy()
        h = self.run_layers(h, pos, range(self.s.L), taps)
        return h, taps

    def truncate(self, length: int) -> None:
        for kv in self.kv:
            kv.length = length

    def prefill_matrix(self, tokens: Sequence[int], all_rows: bool = False):
        """Whole prompt through every layer at once (matrix form of forward_token).

        Returns (final hidden of the last position -- of every position [P, d]
        if `all_rows` --, anchors [P][m] lists).
        """
        P = len(tokens)
        H = np.stack([self.embed(int(t)) for t in tokens])
        taps = [[None] * len(self.s.anchors) for _ in range(P)]
        for p in range(P):
            taps[p][0] = H[p].copy()
        for l in range(self.s.L):
            kv = self.kv[l]
            assert kv.length == 0
            H = layer_matrix(self.s, self.W["layers"][l], H, 0, kv, linear=self.s.linear(l))
            kv.length = P
            if (l + 1) in self.anchor_at:
                for p in range(P):
                    taps[p][self.anchor_at[l + 1]] = H[p].copy()
        return (H.copy() if all_rows else H[-1].copy()), taps


class PDM:
    """Pipeline draft module: FC fusion of anchors, Ls causal decoder layers, own head.

    [PL] §3.1: an Ls-layer Transformer decoder with an independent LM head that
    predicts one token; [RB] method steps 3-4: features of each position are
    the concatenated reachable anchors projected by the FC of its pattern.
    Reading taken: the layers have the target's layer shape with their own
    weights, positions are the true sequence positions, and a final RMSNorm
    precedes the head.
    """

    def __init__(self, w, W):
        self.s = _Shape(w)
        self.W = W
        self.kv = [KVCache(self.s.max_ctx, self.s.Hkv, self.s.hd, self.s.bf16)
                   for _ in range(self.s.Ls)]
        self.C = 0  # committed positions 0..C-1 (features at full depth n)

    def feature(self, taps: Sequence[np.ndarray], k: int) -> np.ndarray:
        """g(p, k) = W_fc[f(k)] * concat(A[p][0..f(k)]) ([RB] core method)."""
        f = pattern(k, self.s.anchors, self.s.L, self.s.n, self.s.split)
        x = np.concatenate([taps[i] for i in range(f + 1)]).astype(F32)
        return self.W["fc"][f] @ x

    def feature_rows(self, taps_rows: Sequence[Sequence[np.ndarray]], k: int) -> np.ndarray:
        """`feature` of many positions at one depth k with one matrix product: [M, d_pdm]."""
        f = pattern(k, self.s.anchors, self.s.L, self.s.n, self.s.split)
        X = np.stack([np.concatenate([taps[i] for i in range(f + 1)]) for taps in taps_rows]).astype(F32)
        return (X @ self.W["fc"][f].T).astype(F32)

    def run_rows(self, G: np.ndarray, pos0: int, matrix: bool = False) -> np.ndarray:
        """All Ls layers over feature rows at positions pos0.. (pos0 == C)."""
        assert pos0 == self.C, "trailing rows must start at the committed length"
        X = G.astype(F32)
        f = layer_matrix if matrix else layer_rows
        for l in range(self.s.Ls):
            X = f(self.s, self.W["pdm_layers"][l], X, pos0, self.kv[l])
        return X

    def logits(self, x: np.ndarray) -> np.ndarray:
        return self.W["pdm_lm_head"] @ rmsnorm(x, self.W["pdm_final_norm"], self.s.eps)

    def commit(self, count: int) -> None:
        self.C += count
        for kv in self.kv:
            kv.length = self.C
