"""CPU check of the grouped GEMM's direct-to-LDS loads (no GPU needed).

tests/gemm_addr_check.cpp enumerates, for one expert FFN call, every
workgroup, wave, lane and load of the six bf16 GEMM launches of its forward
and backward pass (and of the two dgrads run on transposed weights), through the same address functions the kernels use
(csrc/gemm_addr.h), and checks each load against the tensor it reads:
aligned resources below the extent cap, every served load inside its tensor
and at the element the tile needs, every needed element served and
everything else read as zero, LDS destinations inside their stage, and a one
to one map of real tiles onto workgroups.  The group tables below are the
launches the GPU tests and the benchmark make (the five workloads' shapes,
their routed and shared-expert calls) plus edge cases: empty and one-row
groups, partial tiles, 65 groups, round-robin placement, and one group whose
reduction operand spans more than 2 GiB.
"""
import hashlib
import os
import subprocess
import tempfile

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "gemm_addr_check.cpp")
CSRC = os.path.join(ROOT, "mixture_experts_layer_36_amd", "csrc")


def hipcc():
    for c in ("/opt/rocm/bin/hipcc",):
        if os.path.exists(c):
            return c
    pytest.skip("hipcc not available")


@pytest.fixture(scope="module")
def checker():
    h = hashlib.sha256()
    for p in (SRC, os.path.join(CSRC, "gemm_addr.h")):
        h.update(open(p, "rb").read())
    exe = os.path.join(tempfile.gettempdir(), f"moe_gemm_addr_check_{h.hexdigest()[:16]}")
    if not os.path.exists(exe):
        tmp = exe + f".{os.getpid()}"
        subprocess.run([hipcc(), "-x", "hip", "--offload-arch=gfx950", "-O2", "-std=c++17", "-I", CSRC, SRC,
                        "-o", tmp], check=True, capture_output=True)
        os.replace(tmp, exe)
    return exe


def run(exe, d, F, swiglu, offsets, rows_max, rr_R=0, rr_L=1, bounds=None):
    groups = len(offsets) - 1
    text = f"{d} {F} {int(swiglu)} {groups} {rows_max} {rr_R} {rr_L}\n" + " ".join(map(str, offsets)) + "\n"
    if bounds is not None:
        text += f"{len(bounds) - 1}\n" + "\n".join(" ".join(map(str, row)) for row in bounds) + "\n"
    r = subprocess.run([exe], input=text, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0 and r.stdout.startswith("OK"), r.stdout + r.stderr
    return int(r.stdout.split()[1])


def offsets_of(counts):
    return [0] + list(np.cumsum(counts).astype(int))


def near_uniform(total, groups, seed, spread=0.08):
    rng = np.random.default_rng(seed)
    c = rng.uniform(1 - spread, 1 + spread, groups)
    c = np.floor(c / c.sum() * total).astype(int)
    c[0] += total - c.sum()
    return list(c)


CASES = {
    # the five workloads' routed calls (near-uniform counts like their routing)
    "mixtral_routed": dict(d=4096, F=14336, swiglu=True, counts=near_uniform(32768, 8, 1), rows_max=32768),
    "dsv2lite_routed_rr": dict(d=2048, F=1408, swiglu=True, counts=near_uniform(98304, 64, 2), rows_max=98304,
                               rr_R=8, rr_L=8),
    "dsv2lite_shared": dict(d=2048, F=2816, swiglu=True, counts=[16384], rows_max=16384),
    "gpt2s_routed": dict(d=768, F=3072, swiglu=False, counts=near_uniform(16384, 8, 3, 0.03), rows_max=16384),
    "bertl_skew": dict(d=1024, F=4096, swiglu=False,
                       counts=[2048, 2048, 2048, 426, 62, 9, 3, 1] + [0] * 8, rows_max=32768),
    "switch_tiny": dict(d=128, F=256, swiglu=False, counts=[128, 104, 153, 127], rows_max=640),
    # edge cases: empty, one-row and partial tiles; a ragged model width
    "edges": dict(d=64, F=96, swiglu=True, counts=[0, 1, 255, 256, 257, 0, 511, 3], rows_max=1400),
    "ragged_d": dict(d=8200, F=48, swiglu=False, counts=[70, 0, 122, 0], rows_max=192),
    "groups65": dict(d=512, F=512, swiglu=True,
                     counts=[1500] + [(7 * g) % 59 if g % 5 != 1 else 0 for g in range(1, 65)], rows_max=4096),
    # weight-gradient reduction over more than 2 GiB of [dA | dB] (and h)
    "group_over_2gib": dict(d=4096, F=14336, swiglu=True, counts=[40000], rows_max=40000),
}


@pytest.mark.parametrize("name", list(CASES))
def test_every_gemm_load_stays_in_bounds(checker, name):
    c = CASES[name]
    n = run(checker, c["d"], c["F"], c["swiglu"], offsets_of(c["counts"]), c["rows_max"], c.get("rr_R", 0),
            c.get("rr_L", 1))
    assert n > 0


def chunk_bounds(offsets, chunks, seed):
    """Random token-chunk sub-ranges of every group: ascending cut points
    inside each group, some chunks empty."""
    rng = np.random.default_rng(seed)
    G = len(offsets) - 1
    rows = [[offsets[g] for g in range(G)]]
    cuts = [sorted(rng.integers(offsets[g], offsets[g + 1] + 1, chunks - 1)) for g in range(G)]
    for r in range(chunks - 1):
        rows.append([int(cuts[g][r]) for g in range(G)])
    rows.append([offsets[g + 1] for g in range(G)])
    return rows


@pytest.mark.parametrize("name,chunks", [("dsv2lite_routed_rr", 4), ("mixtral_routed", 2), ("edges", 3),
                                         ("bertl_skew", 3)])
def test_gemm_loads_of_token_chunks_stay_in_bounds(checker, name, chunks):
    """The row-split launches of a pipelined step run once per token chunk on
    sub-range group tables (offsets = chunk starts, ends = next chunk's
    starts): every load of every chunk's launches is checked as above."""
    c = CASES[name]
    off = offsets_of(c["counts"])
    n = run(checker, c["d"], c["F"], c["swiglu"], off, c["rows_max"], c.get("rr_R", 0), c.get("rr_L", 1),
            bounds=chunk_bounds(off, chunks, 7 + chunks))
    assert n > 0


def test_the_checker_catches_a_planted_mistake(checker, tmp_path):
    """The same check against a copy of the address header whose stage stride
    is one row short (the kind of slip that reads the wrong K rows) must fail."""
    src = open(os.path.join(CSRC, "gemm_addr.h")).read()
    bad = src.replace("return StageWalk{first, BK * ld_bytes, BK * ld_bytes - col0_bytes};",
                      "return StageWalk{first, (BK - 1) * ld_bytes, BK * ld_bytes - col0_bytes};")
    assert bad != src
    (tmp_path / "gemm_addr.h").write_text(bad)
    exe = str(tmp_path / "check_bad")
    subprocess.run([hipcc(), "-x", "hip", "--offload-arch=gfx950", "-O2", "-std=c++17", "-I", str(tmp_path),
                    SRC, "-o", exe], check=True, capture_output=True)
    text = "64 96 1 2 600 0 1\n0 300 600\n"
    r = subprocess.run([exe], input=text, capture_output=True, text=True, timeout=120)
    assert r.returncode != 0 and r.stdout.startswith("FAIL"), r.stdout
