"""Fill the tensors of a workload from the seeded generator in ``gen.c``.

Tensor ids (mixed into the workload seed): x 1, router weight 2, W1 / W_gate
3, W_up 4, W2 / W_down 5, shared W_gate 6, shared W_up 7, shared W_down 8,
upstream gradient dy 9.

Layouts (row-major):
  x, dy            [T, d]
  w_router         [d, E]
  w1 (or W_gate)   [E, d, ffn];  w_up [E, d, ffn] (SwiGLU only)
  w2 (or W_down)   [E, ffn, d]
  shared weights   the n_shared experts concatenated along the hidden axis:
                   w_gate_s, w_up_s [d, n_shared*ffn_shared],
                   w_down_s [n_shared*ffn_shared, d]; hidden columns
                   [s*ffn_shared, (s+1)*ffn_shared) belong to shared expert s.
  bias             [E] fp32 (only when the workload has a router bias)
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass
from typing import Optional

import numpy as np

from .workloads import Workload, zipf_bias

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libsynth.so")
_lib = None


def build_generator(force: bool = False) -> str:
    """Compile gen.c into libsynth.so next to it (gcc, OpenMP)."""
    if force or not os.path.exists(_SO):
        tmp = _SO + ".tmp"
        subprocess.check_call([
            "gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
            os.path.join(_HERE, "gen.c"), "-o", tmp, "-lm"])
        os.replace(tmp, _SO)
    return _SO


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build_generator()
        lib = ctypes.CDLL(_SO)
        for fn, ptr in (("synth_normal_f32", ctypes.c_void_p),
                        ("synth_normal_bf16", ctypes.c_void_p)):
            f = getattr(lib, fn)
            f.argtypes = [ctypes.c_uint64, ctypes.c_int64, ctypes.c_int64,
                          ctypes.c_double, ctypes.c_double, ptr]
            f.restype = None
        _lib = lib
    return _lib


def normal(seed: int, shape, dtype: str, std: float = 1.0, mean: float = 0.0,
           first: int = 0) -> np.ndarray:
    """Seeded N(mean, std^2) tensor; bf16 is returned as uint16 bit patterns."""
    lib = _load()
    n = int(np.prod(shape)) if len(shape) else 1
    seed &= 0xFFFFFFFFFFFFFFFF
    if dtype == "f32":
        out = np.empty(shape, dtype=np.float32)
        lib.synth_normal_f32(seed, first, n, mean, std, out.ctypes.data)
    elif dtype == "bf16":
        out = np.empty(shape, dtype=np.uint16)
        lib.synth_normal_bf16(seed, first, n, mean, std, out.ctypes.data)
    else:
        raise ValueError(f"unknown dtype {dtype!r}")
    return out


@dataclass
class LayerInputs:
    wl: Workload
    x: np.ndarray
    w_router: np.ndarray
    bias: Optional[np.ndarray]
    w1: np.ndarray
    w_up: Optional[np.ndarray]
    w2: np.ndarray
    ws_gate: Optional[np.ndarray]
    ws_up: Optional[np.ndarray]
    ws_down: Optional[np.ndarray]
    dy: np.ndarray


def _f32_to_storage_exact(a: np.ndarray, dtype: str) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    if dtype == "f32":
        return a
    bits = a.view(np.uint32)
    if np.any(bits & 0xFFFF):
        raise ValueError("value not representable in bf16")
    return (bits >> 16).astype(np.uint16)


def dyadic(seed: int, shape, dtype: str, step: float, lim: float) -> np.ndarray:
    """Seeded values on the grid step*Z, clipped to [-lim, lim]: small
    dyadic numbers whose sums are exact in fp32 (used to force exactly
    equal logits, i.e. ties)."""
    z = normal(seed, shape, "f32", 1.0).astype(np.float64)
    v = np.clip(np.round(z / step) * step, -lim, lim)
    return _f32_to_storage_exact(v, dtype)


def make_inputs(wl: Workload, with_dy: bool = True, dyadic_router: bool = False) -> LayerInputs:
    """Inputs of a workload.  With ``dyadic_router`` the tokens are small
    integers in [-3, 3] and the router weights multiples of 1/2 in [-2, 2]:
    every logit is then exact in fp32 whatever the summation order, and equal
    logits (ties) are frequent."""
    s = wl.seed
    dt = wl.dtype
    T, d, F, E = wl.T, wl.d, wl.ffn, wl.E
    if dyadic_router:
        x = dyadic(s ^ 1, (T, d), dt, 1.0, 3.0)
        w_router = dyadic(s ^ 2, (d, E), dt, 0.5, 2.0)
    else:
        x = normal(s ^ 1, (T, d), dt, 1.0)
        w_router = normal(s ^ 2, (d, E), dt, wl.w_std)
    w1 = normal(s ^ 3, (E, d, F), dt, wl.w_std)
    w_up = normal(s ^ 4, (E, d, F), dt, wl.w_std) if wl.act == "swiglu" else None
    w2 = normal(s ^ 5, (E, F, d), dt, wl.w_std)
    ws_gate = ws_up = ws_down = None
    if wl.n_shared > 0:
        Fs = wl.n_shared * wl.ffn_shared
        ws_gate = normal(s ^ 6, (d, Fs), dt, wl.w_std)
        if wl.act == "swiglu":
            ws_up = normal(s ^ 7, (d, Fs), dt, wl.w_std)
        ws_down = normal(s ^ 8, (Fs, d), dt, wl.w_std)
    bias = None
    if wl.has_bias:
        bias = np.asarray(zipf_bias(E, wl.zipf_s), dtype=np.float64).astype(np.float32)
    dy = normal(s ^ 9, (T, d), dt, 1.0) if with_dy else None
    return LayerInputs(wl, x, w_router, bias, w1, w_up, w2, ws_gate, ws_up,
                       ws_down, dy)
