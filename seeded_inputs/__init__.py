"""Seeded synthetic inputs shared by the CPU oracle and the GPU harness.

This module holds workload shapes, weight / prompt / uniform generators and
dtype plumbing only.  It contains none of the decoding method's arithmetic:
no anchor patterns, no layer math, no schedule.  Both sides of every parity
test read their inputs from here and compute everything else themselves.

Workloads (model shapes follow the 4B / 9B-class targets the pages evaluate
on, with random-init weights, since no trained checkpoint is available):

  tiny_fp32   L=8  d=256  4/4 heads x64   FFN 1024  V=1024   n=4  Ls=1  B=[0,2,4,6,7]
  4b_n8       L=32 d=2560 20/4 heads x128 FFN 9728  V=151936 n=8  Ls=4  B=[0,8,16,24,31]
  9b_n8       L=32 d=4096 32/8 heads x128 FFN 12288 V=151936 n=8  Ls=4  B=[0,8,16,24,31]
  4b_n16      as 4b_n8 but n=16 Ls=2, prompt 4096, 512 new tokens, forced p=0.5
  9b_sample   as 9b_n8, temperature 1.0 rejection-sampling verification

Weights are N(0, 0.02) per linear / embedding matrix (fp32 draws rounded to
bf16 to nearest-even for bf16 models), norm gains are 1 unless asked
otherwise.  Every tensor has its own generator seeded from (workload seed,
tensor index), so a tensor can be regenerated alone.
"""
from __future__ import annotations

import copy
import dataclasses
import hashlib
from typing import Dict, List, Optional

import numpy as np

# Purposes of the per-position uniforms (column index of the uniform table).
U_TARGET, U_DRAFT, U_ACCEPT, U_RESAMPLE, U_FORCE = 0, 1, 2, 3, 4
N_PURPOSES = 5


@dataclasses.dataclass
class Workload:
    name: str
    dtype: str              # "f32" or "bf16": weight and KV-cache storage type
    L: int                  # target decoder layers
    d: int                  # hidden size (the draft module uses the same)
    Hq: int
    Hkv: int
    hd: int
    F: int                  # SwiGLU inner size
    V: int                  # vocabulary
    n: int                  # pipeline stages
    Ls: int                 # draft-module decoder layers
    anchors: List[int]
    P: int                  # prompt length
    G: int                  # tokens to emit (the first comes from prefill)
    mode: str = "greedy"    # "greedy" or "sample"
    policy: str = "natural"  # "natural" or "forced"
    p_accept: float = 0.0   # forced-acceptance probability
    seed: int = 1
    temperature: float = 1.0
    eps: float = 1e-6
    rope_base: float = 10000.0
    norm_gain: str = "ones"  # "ones" or "random" (1 + 0.1 N(0,1), for tests)
    schedule: str = "pre"   # draft-module features: "pre" (before the stage step) or "post"
    top_k: int = 0          # sample mode: keep the k largest logits (0: the whole vocabulary)
    attn_period: int = 0    # hybrid target: layer l is softmax attention iff l % P == P-1, else linear (0: all softmax)
    split: tuple = ()       # layers of stages 0..n-1 (empty: L/n each)
    width: int = 1          # draft-tree width W (1: one draft per cycle)
    p_tree: float = 0.0     # tree forced policy: the true token is among the W candidates w.p. p_tree
                            # (first-ranked w.p. p_accept)

    @property
    def max_ctx(self) -> int:
        # positions reach P+G+n-2 (newest in-flight token) and drafts P+G+n-1
        return self.P + self.G + self.n + 8

    def replace(self, **kw) -> "Workload":
        w = copy.deepcopy(self)
        for k, v in kw.items():
            setattr(w, k, v)
        return w


WORKLOADS: Dict[str, Workload] = {
    "tiny_fp32": Workload("tiny_fp32", "f32", 8, 256, 4, 4, 64, 1024, 1024, 4, 1,
                          [0, 2, 4, 6, 7], P=16, G=64, seed=1),
    "4b_n8": Workload("4b_n8", "bf16", 32, 2560, 20, 4, 128, 9728, 151936, 8, 4,
                      [0, 8, 16, 24, 31], P=512, G=256, policy="forced",
                      p_accept=0.8, seed=2),
    "9b_n8": Workload("9b_n8", "bf16", 32, 4096, 32, 8, 128, 12288, 151936, 8, 4,
                      [0, 8, 16, 24, 31], P=1024, G=256, policy="forced",
                      p_accept=0.7, seed=3),
    "4b_n16": Workload("4b_n16", "bf16", 32, 2560, 20, 4, 128, 9728, 151936, 16, 2,
                       [0, 8, 16, 24, 31], P=4096, G=512, policy="forced",
                       p_accept=0.5, seed=4),
    "9b_sample": Workload("9b_sample", "bf16", 32, 4096, 32, 8, 128, 12288, 151936, 8, 4,
                          [0, 8, 16, 24, 31], P=2048, G=512, mode="sample",
                          temperature=1.0, seed=5),
    # 9b_sample with top-k 50 truncation of P and Q (the pages' evaluation decoding)
    "9b_sample_topk50": Workload("9b_sample_topk50", "bf16", 32, 4096, 32, 8, 128, 12288, 151936, 8, 4,
                                 [0, 8, 16, 24, 31], P=2048, G=512, mode="sample",
                                 temperature=1.0, seed=5, top_k=50),
    # 4b_n8 shapes as a hybrid target: one softmax layer per block of four,
    # the others linear attention
    "4b_hybrid_n8": Workload("4b_hybrid_n8", "bf16", 32, 2560, 20, 4, 128, 9728, 151936, 8, 4,
                             [0, 8, 16, 24, 31], P=512, G=256, policy="forced",
                             p_accept=0.8, seed=6, attn_period=4),
    # 4b_n8 with the draft module on post-step features (scheduling ablation)
    "4b_n8_post": Workload("4b_n8_post", "bf16", 32, 2560, 20, 4, 128, 9728, 151936, 8, 4,
                           [0, 8, 16, 24, 31], P=512, G=256, policy="forced",
                           p_accept=0.8, seed=2, schedule="post"),
    # 4b_n8 with a width-4 draft tree: the true token is the best-ranked
    # candidate w.p. 0.8 (as in 4b_n8) and among the 4 w.p. 0.87 -- the tree
    # acceptance the pages' width-4 results imply (n=8 theoretical speedup
    # 3.05 -> 3.84, i.e. a reject rate ~0.67x that of one draft)
    "4b_tree4_n8": Workload("4b_tree4_n8", "bf16", 32, 2560, 20, 4, 128, 9728, 151936, 8, 4,
                            [0, 8, 16, 24, 31], P=512, G=256, policy="forced",
                            p_accept=0.8, seed=2, width=4, p_tree=0.87),
    # 4B shapes on the pages' non-uniform 4-stage split 5+4;9;9;9 (a 5-layer
    # first stage, three 9-layer stages, a 4-layer draft module)
    "4b_split_n4": Workload("4b_split_n4", "bf16", 32, 2560, 20, 4, 128, 9728, 151936, 4, 4,
                            [0, 8, 16, 24, 31], P=512, G=256, policy="forced",
                            p_accept=0.8, seed=7, split=(5, 9, 9, 9)),
}


def workload(name: str, **overrides) -> Workload:
    return WORKLOADS[name].replace(**overrides)


def _tensor_seed(seed: int, index: int) -> int:
    h = hashlib.blake2b(f"spd-weights/{seed}/{index}".encode(), digest_size=8).digest()
    return int.from_bytes(h, "little") & 0x7FFF_FFFF_FFFF_FFFF


def tensor_specs(w: Workload):
    """(name, shape, kind) for every model tensor, in generator-index order.

    Layouts (row-major, output features first):
      embed [V, d]; w_qkv [(Hq+2Hkv)*hd, d] (q rows, then k, then v);
      w_o [d, Hq*hd]; w_gu [2F, d] (gate rows 0..F-1, up rows F..2F-1);
      w_down [d, F]; lm_head [V, d]; fc[f] [d, (f+1)*d] (input = anchors 0..f
      concatenated in anchor order); norms [d] (always fp32).
    """
    specs = [("embed", (w.V, w.d), "mat")]

    def layer(prefix):
        return [
            (prefix + "attn_norm", (w.d,), "norm"),
            (prefix + "w_qkv", ((w.Hq + 2 * w.Hkv) * w.hd, w.d), "mat"),
            (prefix + "w_o", (w.d, w.Hq * w.hd), "mat"),
            (prefix + "ffn_norm", (w.d,), "norm"),
            (prefix + "w_gu", (2 * w.F, w.d), "mat"),
            (prefix + "w_down", (w.d, w.F), "mat"),
        ]

    for i in range(w.L):
        specs += layer(f"layers.{i}.")
    specs += [("final_norm", (w.d,), "norm"), ("lm_head", (w.V, w.d), "mat")]
    for f in range(len(w.anchors)):
        specs.append((f"fc.{f}", (w.d, (f + 1) * w.d), "mat"))
    for i in range(w.Ls):
        specs += layer(f"pdm_layers.{i}.")
    specs += [("pdm_final_norm", (w.d,), "norm"), ("pdm_lm_head", (w.V, w.d), "mat")]
    return specs


def make_weights(w: Workload, device: str = "cpu"):
    """Generate every model tensor with torch's seeded generator on `device`.

    Returns {name: torch.Tensor}; matrices are bf16 or fp32 (per w.dtype),
    norm gains fp32.  CPU and GPU generators give different values for the
    same seed; within one test both sides always read the same tensors.
    """
    import torch

    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    out = {}
    for idx, (name, shape, kind) in enumerate(tensor_specs(w)):
        g = torch.Generator(device=device)
        g.manual_seed(_tensor_seed(w.seed, idx))
        if kind == "norm":
            if w.norm_gain == "ones":
                t = torch.ones(shape, dtype=torch.float32, device=device)
            else:
                t = 1.0 + 0.1 * torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        else:
            t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
            t.mul_(0.02)
            t = t.to(dt)
        out[name] = t.contiguous()
    return out


def weights_numpy_f32(tensors) -> Dict[str, np.ndarray]:
    """Upcast every tensor to a host float32 numpy array (exact for bf16)."""
    import torch

    out = {}
    for k, t in tensors.items():
        out[k] = t.detach().to("cpu", torch.float32).numpy().copy()
    return out


def nest_weights(flat: Dict[str, np.ndarray], w: Workload) -> dict:
    """Group a flat {name: array} dict into the nested model dict both sides use."""
    def layer(prefix):
        return {k: flat[prefix + k] for k in
                ("attn_norm", "w_qkv", "w_o", "ffn_norm", "w_gu", "w_down")}
    return {
        "embed": flat["embed"],
        "layers": [layer(f"layers.{i}.") for i in range(w.L)],
        "final_norm": flat["final_norm"],
        "lm_head": flat["lm_head"],
        "fc": [flat[f"fc.{f}"] for f in range(len(w.anchors))],
        "pdm_layers": [layer(f"pdm_layers.{i}.") for i in range(w.Ls)],
        "pdm_final_norm": flat["pdm_final_norm"],
        "pdm_lm_head": flat["pdm_lm_head"],
    }


def make_prompt(w: Workload, seed: Optional[int] = None) -> np.ndarray:
    """Prompt token ids, uniform in [0, V), int32."""
    s = w.seed if seed is None else seed
    rng = np.random.Generator(np.random.Philox(key=[s, 0x5052]))
    return rng.integers(0, w.V, size=w.P, dtype=np.int64).astype(np.int32)


def make_uniforms(w: Workload, seed: Optional[int] = None) -> np.ndarray:
    """Per-position uniforms [max_ctx, N_PURPOSES], float32 multiples of 2^-24.

    Column j is keyed by purpose (TARGET, DRAFT, ACCEPT, RESAMPLE, FORCE) and
    row p by the position the draw decides, so the same draw is seen whatever
    the schedule.  Values k * 2^-24 are exact in fp32 and fp64.
    """
    s = w.seed if seed is None else seed
    rng = np.random.Generator(np.random.Philox(key=[s, 0x554E]))
    k = rng.integers(0, 1 << 24, size=(w.max_ctx, N_PURPOSES), dtype=np.int64)
    return (k.astype(np.float64) * 2.0 ** -24).astype(np.float32)


def tiny(name: str = "t", **kw) -> Workload:
    """A small workload for tests: defaults sized so the oracle runs in seconds."""
    base = dict(name=name, dtype="f32", L=4, d=64, Hq=4, Hkv=2, hd=16, F=96, V=97,
                n=2, Ls=1, anchors=[0, 2, 3], P=5, G=12, seed=11)
    base.update(kw)
    return Workload(**base)
