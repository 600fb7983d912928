"""ctypes view of libmoe's C ABI (include/moe.h).

Loads the in-tree libmoe.so.  There is no fallback: if the library has not
been built, loading raises and nothing runs.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe.so")

MOE_OK, MOE_ERR_INVALID, MOE_ERR_UNSUPPORTED, MOE_ERR_HIP = 0, -1, -2, -3
DTYPES = {"f32": 0, "bf16": 1}
GATINGS = {"softmax_topk": 0, "softmax_topk_renorm": 1, "topk_softmax": 2}
ACTS = {"gelu": 0, "swiglu": 1}
PLACEMENTS = {"contiguous": 0, "round_robin": 1}


class MoeConfig(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int64), ("d", ctypes.c_int64), ("ffn", ctypes.c_int64),
        ("E", ctypes.c_int64), ("k", ctypes.c_int64),
        ("capacity_factor", ctypes.c_float),
        ("gating", ctypes.c_int32), ("act", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("ep_ranks", ctypes.c_int32), ("placement", ctypes.c_int32),
        ("n_shared", ctypes.c_int64), ("ffn_shared", ctypes.c_int64),
    ]


class MoeSizes(ctypes.Structure):
    _fields_ = [("C", ctypes.c_int64), ("n_max", ctypes.c_int64),
                ("workspace_bytes", ctypes.c_size_t)]


class MoeGroups(ctypes.Structure):
    _fields_ = [("groups", ctypes.c_int64), ("ffn", ctypes.c_int64),
                ("rows_max", ctypes.c_int64), ("offsets", ctypes.c_void_p),
                ("use_placement", ctypes.c_int32), ("ends", ctypes.c_void_p)]


_P = ctypes.c_void_p
_CFG = ctypes.POINTER(MoeConfig)
_GRP = ctypes.POINTER(MoeGroups)

SIGNATURES = {
    "moe_plan": [_CFG, ctypes.POINTER(MoeSizes)],
    "moe_route": [_CFG, _P, _P, _P, _P, _P, _P, _P, _P],
    "moe_dispatch": [_CFG, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P],
    "moe_dispatch_noalloc": [_CFG, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P],
    "moe_expert_ffn_fwd": [_CFG, _GRP, _P, _P, _P, _P, _P, _P, _P, _P],
    "moe_expert_ffn_bwd": [_CFG, _GRP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P],
    "moe_expert_ffn_bwd_data": [_CFG, _GRP, _P, _P, _P, _P, _P, _P, _P, _P],
    "moe_expert_ffn_bwd_weights": [_CFG, _GRP, _P, _P, _P, _P, _P, _P, _P, _P],
    "moe_permute": [_CFG, _P, _P, _P, _P],
    "moe_expert_ffn_fwd_fused": [_CFG, _GRP, _P, _P, _P, _P, _P, _P, _P, _P, _P],
    "moe_combine_fused": [_CFG, _P, _P, _P, _P, _P],
    "moe_chunk_rows": [_CFG, _P, _P, _P, ctypes.c_int64, ctypes.POINTER(ctypes.c_int64), _P, _P],
    "moe_combine": [_CFG, _P, _P, _P, _P, _P, _P],
    "moe_combine_bwd": [_CFG, _P, _P, _P, _P, _P, _P, _P],
    "moe_route_bwd": [_CFG, _P, _P, _P, _P, _P, _P, _P, _P, _P],
    "moe_aux_loss": [_CFG, _P, _P, ctypes.c_float, _P, _P, _P],
    "moe_aux_loss_bwd": [_CFG, _P, _P, ctypes.c_float, _P, _P],
    "moe_dispatch_bwd": [_CFG, _P, _P, _P, _P, _P, _P, _P],
    "moe_status_string": [ctypes.c_int],
    "moe_last_hip_error": [],
}

_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"libmoe.so is not built ({LIB_PATH}); run "
                "`python -m mixture_experts_layer_36_amd.build` first")
        lib = ctypes.CDLL(LIB_PATH)
        for name, args in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = ctypes.c_char_p if name == "moe_status_string" else ctypes.c_int
        _lib = lib
    return _lib


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        lib = load()
        msg = lib.moe_status_string(status).decode()
        extra = f" (hipError {lib.moe_last_hip_error()})" if status == MOE_ERR_HIP else ""
        super().__init__(f"{fn}: {msg}{extra}")
        self.status = status


def call(name: str, *args) -> None:
    st = getattr(load(), name)(*args)
    if st != MOE_OK:
        raise MoeError(name, st)


def make_config(T, d, ffn, E, k, capacity_factor, gating, act, dtype,
                ep_ranks=1, placement="contiguous", n_shared=0, ffn_shared=0) -> MoeConfig:
    return MoeConfig(T=T, d=d, ffn=ffn, E=E, k=k, capacity_factor=float(capacity_factor),
                     gating=GATINGS[gating] if isinstance(gating, str) else gating,
                     act=ACTS[act] if isinstance(act, str) else act,
                     dtype=DTYPES[dtype] if isinstance(dtype, str) else dtype,
                     ep_ranks=ep_ranks,
                     placement=PLACEMENTS[placement] if isinstance(placement, str) else placement,
                     n_shared=n_shared, ffn_shared=ffn_shared)


def plan(cfg: MoeConfig) -> MoeSizes:
    out = MoeSizes()
    call("moe_plan", ctypes.byref(cfg), ctypes.byref(out))
    return out
