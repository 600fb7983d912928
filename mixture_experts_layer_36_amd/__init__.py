"""libmoe: one GPU's share of a mixture-of-experts layer on AMD MI355X (gfx950).

The computation lives in hand-written HIP kernels behind the C ABI of
include/moe.h (libmoe.so, built by ``mixture_experts_layer_36_amd.build``);
this package is the ctypes binding (``api``: one function per entry point)
and a layer runner that owns the buffers (``layer.MoELayer``).
"""
from . import _native  # noqa: F401
from ._native import MoeConfig, MoeError, MoeGroups, MoeSizes, make_config, plan  # noqa: F401

__all__ = ["MoeConfig", "MoeError", "MoeGroups", "MoeSizes", "make_config", "plan"]
