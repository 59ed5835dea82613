"""MI355X-native sparse Mixture-of-Experts FFN layer forward.

The layer runs in hand-written HIP kernels for gfx950 behind the C ABI of include/moe.h
(libmoe.so, built in-tree by ``python -m sparse_mixture_experts_41_amd.build``); ``ops`` is the
torch-facing binding (argument marshalling only). There is no CPU fallback: calling into the
layer without the built library raises.
"""
from ._lib import LIB_PATH, MoeConfig, MoeError, load, make_config

__all__ = ["LIB_PATH", "MoeConfig", "MoeError", "load", "make_config"]
