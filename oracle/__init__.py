"""CPU oracle for the speculative-pipeline-decoding (SPD) cycle.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package; only tests/, the smoke check and the benchmark's CPU
baseline leg do.  It shares no code with the HIP library: it reads its inputs
from `seeded_inputs` and computes everything else itself, in plain numpy
float32 (float64 where a sampling decision is taken), one token and one layer
at a time.

Citation tags used in this package (section names are those on each page):
  [RB] paper.rainbus.top summary of arXiv 2605.30852, "Speculative Pipeline
       Decoding: Higher-Accuracy and Zero-Bubble Speculation via Pipeline
       Parallelism" (Chinese structured summary): sections "core method",
       "method steps" (steps 1-6), "technical novelty".
  [TW] techwalker.com article on the same paper (Chinese news write-up),
       sections 3 (pipeline), 4 (multi-depth fusion), 5 (simultaneous
       execution), 6 (verification and rollback), 8 (speedup metric).
  [PL] paperlayer.ai summary of arXiv 2605.30852v3, "Speculative Pipeline
       Decoding: Higher-Accuracy Drafting with Hidden Latency via Pipeline
       Parallelism": sections 3.1-3.4, A.1-A.3.
  [YB] ybb.press blog "Breaking the autoregressive bottleneck: speculative
       decoding ..." (generic, not about SPD), sections 2.1-2.2 (rejection
       sampling rule and its lossless identity).

Parity status of each function is stated in its docstring: every function is
pinned by a CPU test (tests/test_oracle_*.py) against a closed form, a page's
worked example, an independent library routine or brute force.
"""
from .schedule import (lmax, pattern, pattern_table, n_patterns, stage_layers,
                       depth_layout, key_depth, cycle_count, validate_shape)
from .layers import bf16_round, rmsnorm, rope_cos_sin, apply_rope, attention, silu
from .model import Target, PDM, KVCache
from .spd import SPDOracle, ar_greedy, ForcedPolicy, NaturalPolicy
from . import sampling

__all__ = [
    "lmax", "pattern", "pattern_table", "n_patterns", "stage_layers", "depth_layout",
    "key_depth", "cycle_count", "validate_shape", "bf16_round", "rmsnorm",
    "rope_cos_sin", "apply_rope", "attention", "silu", "Target", "PDM", "KVCache",
    "SPDOracle", "ar_greedy", "ForcedPolicy", "NaturalPolicy", "sampling",
]
