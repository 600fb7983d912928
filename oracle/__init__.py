"""CPU oracle for the MoE layer — TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct float64 numpy implementation of what the
GPU path computes.  Only the tests, the smoke check and the CPU-baseline leg
of the benchmark may import it; the product path (the HIP library and its
Python binding) never does and shares no code with it.

Every function cites the passage of the pages it follows: the tutorial
chapter "第 4 章 … 扩展 MoE 模型——迈向分布式训练" (sections on expert
parallelism, EP+DP training, the all-to-all pattern, the frameworks), the
Piper summary (resource model: routing table and expert capacity) and the
FSMoE abstract (routing, communication, expert computation modules).  Where
the pages leave a step open, the reading adopted is stated in the docstring.

Pinned by tests/test_oracle_*.py against brute force, closed forms, the
pages' worked example, invariants, a dense-masked evaluation, float64 finite
differences and torch CPU autograd.  Nothing here is "parity unpinned".
"""
from .moe import *  # noqa: F401,F403
