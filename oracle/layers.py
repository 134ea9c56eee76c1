"""Decoder-layer primitives of the target and draft module (test infrastructure only).

The pages name the layer family (GQA attention over a per-layer KV cache,
RMSNorm, SwiGLU, RoPE) but not its constants; the readings taken are:
rotate-half RoPE with theta_i = base^(-2i/hd), base 10000; RMSNorm
x / sqrt(mean(x^2) + eps) * gamma with eps = 1e-6; no biases; no QK-norm.
All arithmetic is float32 numpy, one token at a time.
"""
from __future__ import annotations

import numpy as np

F32 = np.float32


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even), returned as float32.

    Models the storage of the KV cache in bf16 models.  Pinned against
    torch's float32 -> bfloat16 conversion in the CPU tests.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return r.view(np.float32).reshape(np.shape(x))


def rmsnorm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * gamma, float32."""
    x = x.astype(F32, copy=False)
    ms = np.mean(x * x, dtype=F32)
    return (x / np.sqrt(ms + F32(eps))) * gamma


def silu(x: np.ndarray) -> np.ndarray:
    return x / (F32(1) + np.exp(-x))


def rope_cos_sin(pos: int, hd: int, base: float):
    """cos/sin of pos * theta_i, theta_i = base^(-2i/hd), i < hd/2 (fp64, rounded to fp32)."""
    i = np.arange(hd // 2, dtype=np.float64)
    theta = np.power(np.float64(base), -2.0 * i / hd)
    ang = np.float64(pos) * theta
    return np.cos(ang).astype(F32), np.sin(ang).astype(F32)


def rope_tables(positions, hd: int, base: float):
    """`rope_cos_sin` for many positions at once: cos, sin [len(positions), hd/2].

    The same fp64 operations per element, so the values are identical.
    """
    i = np.arange(hd // 2, dtype=np.float64)
    theta = np.power(np.float64(base), -2.0 * i / hd)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * theta[None, :]
    return np.cos(ang).astype(F32), np.sin(ang).astype(F32)


def apply_rope(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate-half RoPE on the last axis: pairs (i, i + hd/2) rotate by angle i."""
    h = x.shape[-1] // 2
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1).astype(F32)


def attention(q: np.ndarray, K: np.ndarray, V: np.ndarray) -> np.ndarray:
    """Grouped-query attention of one query position over keys K, V.

    q [Hq, hd]; K, V [T, Hkv, hd]; query head h reads kv head h // (Hq/Hkv).
    softmax(q.k / sqrt(hd)) v per head, float32.
    """
    Hq, hd = q.shape
    Hkv = K.shape[1]
    grp = Hq // Hkv
    scale = F32(1.0 / np.sqrt(hd))
    out = np.empty((Hq, hd), dtype=F32)
    for h in range(Hq):
        kv = h // grp
        s = (K[:, kv, :] @ q[h]) * scale
        s = s - s.max()
        p = np.exp(s)
        p = p / p.sum(dtype=F32)
        out[h] = p @ V[:, kv, :]
    return out


def elu_plus_one(x: np.ndarray) -> np.ndarray:
    """phi(x) = elu(x) + 1: x + 1 for x > 0, exp(x) otherwise (> 0 everywhere)."""
    x = np.asarray(x, F32)
    return np.where(x > 0, x + F32(1), np.exp(np.minimum(x, F32(0)))).astype(F32)


def linear_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray) -> np.ndarray:
    """Causal linear attention of one query position over keys K, V.

    The hybrid target's linear layers (reading: the textbook kernelised
    attention, with feature map phi = elu + 1): query head h reads kv head
    h // (Hq/Hkv) and returns sum_i w_i v_i / sum_i w_i with weights
    w_i = phi(q_h) . phi(k_i) in place of the softmax scores -- no scale, no
    normalisation beyond the weight sum.  q [Hq, hd]; K, V [T, Hkv, hd].
    """
    Hq, hd = q.shape
    Hkv = K.shape[1]
    grp = Hq // Hkv
    out = np.empty((Hq, hd), dtype=F32)
    pk = elu_plus_one(K)
    for h in range(Hq):
        kv = h // grp
        w = pk[:, kv, :] @ elu_plus_one(q[h])
        out[h] = (w @ V[:, kv, :]) / w.sum(dtype=F32)
    return out
