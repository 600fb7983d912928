"""GPU parity of the router backward (moe_route_bwd) against the oracle,
through the C ABI, over the launch shapes of its kernels.

moe_route_bwd forms dlogits through the gating Jacobian (plus an optional
second gradient of the logits) and dW_r = x^T dlogits (tutorial ch.4,
专家并行与数据并行的结合 三.4: the replicated gate's gradients), the latter
as per-token-block partials and a fixed-order sum of them.  For bf16 x the
partials come from the bf16 matrix cores, with experts padded to 16, 32 or
64 and workgroups of 8, 4 or 2 waves owning 512, 256 or 128 columns: the
widest whose column blocks times the token blocks (T / 128, at most 64) give
each of 256 CUs a workgroup.  The cases below reach every padding and width
(the width each one takes on a 256-CU device is named), with ragged T, d
that ends inside a column block, E that is not a multiple of 4, k from 1 to
8, the three gating modes, and the optional added gradient.  fp32 x runs the
fp32 matrix-core kernel.

Bars (max|err| / max|ref| against the float64 oracle on the same inputs):
dlogits 1e-5 (fp32 arithmetic); dW_r 4e-3 for bf16 x (its bf16 rounding is
2^-9 relative; dlogits enter as bf16 hi + lo, about 16 bits) and 1e-5 for
fp32 x, both against the oracle's own dlogits and against x^T times the
GPU's dlogits.  Two runs give bit-identical outputs.  With one token, each
element of dW_r is a single product x_i dl_e, which the hi + lo split
carries to about 2^-17: it must be the bf16 rounding of the exact product
within one unit in the last place, and exactly that rounding for at least
99% of the elements (a split that lost its low half, or a bf16 dl, would
round about half of them differently).
"""
import os
import sys

import numpy as np
import pytest
import torch

import oracle
from synth.tensors import normal
from mixture_experts_layer_36_amd import _native, api
from mixture_experts_layer_36_amd._native import make_config, plan

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

from gpu_helpers import bits, dev, host, rel_err  # noqa: E402

TOL_DL = 1e-5
TOL_DW = {"bf16": 4e-3, "f32": 1e-5}


@pytest.fixture(scope="module", autouse=True)
def native_lib():
    if not os.path.exists(_native.LIB_PATH):
        pytest.fail("libmoe.so is not built; build it before running GPU tests")
    _native.load()


# name: (T, d, E, k, gating, dtype, with an added logits gradient, seed)
CASES = {
    # 16 padded experts, 8 waves (5 column blocks, the last one 8 columns wide)
    "T8192_d2056_E16_add": (8192, 2056, 16, 2, "softmax_topk", "bf16", True, 301),
    # 16 padded, 8 waves: the Mixtral router shape
    "T16384_d4096_E8": (16384, 4096, 8, 2, "topk_softmax", "bf16", False, 302),
    # 16 padded, 4 waves (3 blocks of 512 would leave CUs idle)
    "T9000_d1032_E12": (9000, 1032, 12, 3, "softmax_topk_renorm", "bf16", False, 303),
    # 16 padded, 2 waves: the GPT-2 router shape
    "T8191_d768_E8_add": (8191, 768, 8, 2, "softmax_topk_renorm", "bf16", True, 304),
    # 16 padded, 2 waves; 5 experts, few token blocks
    "T1000_d200_E5": (1000, 200, 5, 2, "topk_softmax", "bf16", False, 305),
    # 32 padded, 8 waves
    "T16384_d2048_E20": (16384, 2048, 20, 4, "softmax_topk", "bf16", True, 306),
    # 32 padded, 2 waves; k = 8
    "T777_d520_E32_k8": (777, 520, 32, 8, "softmax_topk_renorm", "bf16", False, 307),
    # 64 padded, 8 waves: the DeepSeek-V2-Lite router shape
    "T16384_d2048_E64": (16384, 2048, 64, 6, "softmax_topk", "bf16", False, 308),
    # 64 padded, 4 waves
    "T8192_d1024_E64_add": (8192, 1024, 64, 6, "topk_softmax", "bf16", True, 309),
    # 64 padded, 2 waves; 40 experts, top-1
    "T300_d64_E40_k1": (300, 64, 40, 1, "softmax_topk", "bf16", False, 310),
    # one token, one 8-wide piece of d
    "T1_d8_E2": (1, 8, 2, 2, "softmax_topk_renorm", "bf16", False, 311),
    # fp32 x: the fp32 matrix-core kernel
    "T3000_d136_E24_f32_add": (3000, 136, 24, 2, "softmax_topk", "f32", True, 312),
    "T513_d64_E64_f32": (513, 64, 64, 3, "topk_softmax", "f32", False, 313),
}


def run_case(T, d, E, k, gating, dtype, with_add, seed):
    x = normal(seed * 11 + 1, (T, d), dtype, 1.0)
    logits = normal(seed * 11 + 2, (T, E), "f32", 2.0)
    idx = oracle.select_topk(logits.astype(np.float64), k).astype(np.int32)
    dg = normal(seed * 11 + 3, (T, k), "f32", 1.0)
    add = normal(seed * 11 + 4, (T, E), "f32", 0.1) if with_add else None
    cfg = make_config(T, d, 16, E, k, 0.0, gating, "gelu", dtype)
    ws_bytes = plan(cfg).workspace_bytes
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    out = dict(x=dev(x), logits=dev(logits), idx=dev(idx), dg=dev(dg), add=dev(add),
               dl=torch.empty(T, E, dtype=torch.float32, device="cuda"),
               dw=torch.empty(d, E, dtype=tdt, device="cuda"),
               ws=torch.empty(max(256, (ws_bytes + 255) // 256 * 256), dtype=torch.uint8, device="cuda"))

    def call():
        api.moe_route_bwd(cfg, out["x"], out["logits"], out["idx"], out["dg"], out["add"], out["dl"],
                          out["dw"], out["ws"])
    return call, out, x, logits, idx, dg, add


def bf16_round(a: np.ndarray) -> np.ndarray:
    """float64 -> nearest bf16 (ties to even), via float32, as float64."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def bf16_ulp(a: np.ndarray) -> np.ndarray:
    """Unit in the last place of bf16 values (8 significant bits)."""
    _, e = np.frexp(a)
    return np.where(a == 0.0, 2.0 ** -133, np.ldexp(1.0, e - 8))


@pytest.mark.parametrize("name", list(CASES))
def test_route_bwd_parity(name):
    T, d, E, k, gating, dtype, with_add, seed = CASES[name]
    print(f"\n[case] route_bwd {name}", flush=True)
    sys.stdout.flush()
    call, out, x, logits, idx, dg, add = run_case(T, d, E, k, gating, dtype, with_add, seed)
    call()
    torch.cuda.synchronize()
    dl_ref = oracle.gating_backward(logits.astype(np.float64), idx, dg.astype(np.float64), gating)
    if add is not None:
        dl_ref = dl_ref + add.astype(np.float64)
    g_dl = host(out["dl"])
    e = rel_err(g_dl, dl_ref)
    assert np.all(np.isfinite(g_dl)) and e <= TOL_DL, f"dlogits: {e:.3e}"

    x64 = oracle.to_f64(x)
    dummy_w = np.zeros((d, E))
    dw_ref, _ = oracle.router_backward(x64, dummy_w, dl_ref)
    dw_own, _ = oracle.router_backward(x64, dummy_w, g_dl)
    g_dw = host(out["dw"])
    assert np.all(np.isfinite(g_dw))
    e1, e2 = rel_err(g_dw, dw_ref), rel_err(g_dw, dw_own)
    assert e1 <= TOL_DW[dtype], f"dw_router against the oracle's dlogits: {e1:.3e}"
    assert e2 <= TOL_DW[dtype], f"dw_router against x^T (GPU dlogits): {e2:.3e}"

    # deterministic: a second call gives the same bits
    l1, w1 = bits(out["dl"]).copy(), bits(out["dw"]).copy()
    out["dl"].fill_(float("nan"))
    out["dw"].fill_(float("nan"))
    out["ws"].fill_(0xFF)
    call()
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(out["dl"]), l1)
    np.testing.assert_array_equal(bits(out["dw"]), w1)


@pytest.mark.parametrize("d,E", [(2056, 16), (520, 20), (1024, 64)])
def test_route_bwd_single_token_products(d, E):
    print(f"\n[case] route_bwd one token d={d} E={E}", flush=True)
    call, out, x, logits, idx, dg, add = run_case(1, d, E, 2, "softmax_topk", "bf16", True, 320 + E)
    call()
    torch.cuda.synchronize()
    g_dl = host(out["dl"])
    prod = oracle.router_backward(oracle.to_f64(x), np.zeros((d, E)), g_dl)[0]  # exact in float64
    r = bf16_round(prod)
    g_dw = host(out["dw"])
    off = np.abs(g_dw - r)
    assert np.all(off <= bf16_ulp(r)), f"dw_router: {np.max(off / bf16_ulp(r)):.2f} ulp from the rounded product"
    share = np.count_nonzero(off) / off.size
    assert share <= 0.01, f"dw_router: {share:.2%} of the elements off the rounded product"
