"""Seeded synthetic inputs for the MoE layer workloads.

This package is shared by the GPU path's tests/bench and by the CPU oracle.
It describes the workloads (shapes, dtypes, distributions) and fills tensors
with seeded normal numbers; it contains none of the MoE method's arithmetic
(no routing, no capacity rule, no FFN).  Values are produced by the
counter-based SplitMix64 + Box-Muller generator in ``gen.c`` and returned as
numpy arrays: fp32 tensors as ``float32``, bf16 tensors as their raw 16-bit
patterns in ``uint16`` arrays.
"""
from .workloads import WORKLOADS, Workload, workload, zipf_bias  # noqa: F401
from .tensors import LayerInputs, dyadic, make_inputs, normal  # noqa: F401
