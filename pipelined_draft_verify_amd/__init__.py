"""MI355X-native speculative pipeline decoding (SPD): one-GPU SPD cycle.

`libspd.so` (HIP, gfx950) implements the cycle behind the C ABI of
include/spd.h; `_abi` mirrors that ABI with same-named ctypes wrappers and
`engine.SPDEngine` supplies device memory and streams from PyTorch.
"""
from . import _abi
from ._abi import SPDError, lib
from .engine import REC_DTYPE, SPDEngine, make_config, make_weights_struct

__all__ = ["_abi", "SPDError", "lib", "REC_DTYPE", "SPDEngine", "make_config", "make_weights_struct"]
