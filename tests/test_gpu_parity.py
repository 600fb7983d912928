"""GPU parity of libmoe against the CPU oracle, through the C ABI.

Bars (per tensor, max|err| / max|ref|): 1e-5 for fp32 workloads, 2e-2 for
bf16 against the float64 oracle on the same bf16 inputs; logits 1e-5 in both.
Routing indices, counts, offsets, send layout, row maps and the permuted rows
are compared bit for bit, with the oracle routing on the GPU's own fp32
logits.  Every workload is compared element by element: the three smaller
ones here, the Mixtral- and DeepSeek-V2-Lite-shaped ones expert by expert in
test_gpu_large.py.  The expert rows' hidden activation h and the saved
factors of its derivative (act_saved: GELU'(Z), or dh/dA | dh/dB) are
compared too, against oracle.activation_factors of the oracle's own forward.
"""
import os
import sys

import numpy as np
import pytest
import torch

import synth
from mixture_experts_layer_36_amd import _native

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

from gpu_helpers import TOL, bits, host, make_layer, run_full_parity  # noqa: E402


def announce(name):
    print(f"\n[case] {name}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def native_lib():
    if not os.path.exists(_native.LIB_PATH):
        pytest.fail("libmoe.so is not built; build it before running GPU tests")
    _native.load()


@pytest.mark.parametrize("name", ["switch_tiny_f32", "gpt2s_bf16", "bertl_skew_bf16"])
def test_workload_full(name):
    announce(name)
    wl = synth.workload(name)
    inp = synth.make_inputs(wl)
    _, ref, errs = run_full_parity(wl, inp)
    print({k: f"{v:.2e}" for k, v in errs.items()}, "n =", ref["layout"]["n"], flush=True)


W = synth.Workload
FUZZ = {
    "T1_E1_f32": W("T1_E1_f32", T=1, d=8, ffn=8, E=1, k=1, capacity_factor=1.0,
                   gating="softmax_topk", act="gelu", dtype="f32", seed=11),
    "T63_E3_swiglu_drops": W("T63_E3_swiglu_drops", T=63, d=72, ffn=24, E=3, k=2, capacity_factor=0.5,
                             gating="softmax_topk_renorm", act="swiglu", dtype="bf16", seed=12),
    "T64_kE_f32_swiglu": W("T64_kE_f32_swiglu", T=64, d=128, ffn=136, E=4, k=4, capacity_factor=0.0,
                           gating="topk_softmax", act="swiglu", dtype="f32", seed=13),
    "T65_E16_C1": W("T65_E16_C1", T=65, d=64, ffn=256, E=16, k=3, capacity_factor=0.01,
                    gating="softmax_topk", act="gelu", dtype="bf16", seed=14),
    "T1000_E64_rr_shared": W("T1000_E64_rr_shared", T=1000, d=72, ffn=1408, E=64, k=6,
                             capacity_factor=0.0, gating="softmax_topk", act="swiglu", dtype="bf16",
                             ep_ranks=8, placement="round_robin", n_shared=2, ffn_shared=24, seed=15),
    "T300_E8_bias": W("T300_E8_bias", T=300, d=128, ffn=64, E=8, k=2, capacity_factor=1.0,
                      gating="softmax_topk_renorm", act="gelu", dtype="bf16", zipf_s=1.2, seed=16),
    "T257_E2_f32_drops": W("T257_E2_f32_drops", T=257, d=96, ffn=40, E=2, k=1, capacity_factor=0.9,
                           gating="softmax_topk", act="gelu", dtype="f32", seed=17),
    "T512_kE8_swiglu": W("T512_kE8_swiglu", T=512, d=64, ffn=64, E=8, k=8, capacity_factor=0.0,
                         gating="softmax_topk_renorm", act="swiglu", dtype="bf16", seed=18),
    "T777_E32_rr_f32": W("T777_E32_rr_f32", T=777, d=200, ffn=96, E=32, k=5, capacity_factor=1.3,
                         gating="topk_softmax", act="gelu", dtype="f32", ep_ranks=4,
                         placement="round_robin", seed=19),
    "T2000_E5_f32_shared": W("T2000_E5_f32_shared", T=2000, d=40, ffn=48, E=5, k=2, capacity_factor=1.1,
                             gating="softmax_topk", act="swiglu", dtype="f32", n_shared=1,
                             ffn_shared=16, seed=20),
    # every expert-count specialisation of the routing / router-backward /
    # un-permute kernels: E equal to its padded width (8, 16, 32, 64) and E
    # below it, for both dtypes, with top-k at most 2 and above 2
    "T129_E32_bf16": W("T129_E32_bf16", T=129, d=136, ffn=72, E=32, k=3, capacity_factor=1.2,
                       gating="softmax_topk", act="gelu", dtype="bf16", seed=21),
    "T200_E8_f32": W("T200_E8_f32", T=200, d=64, ffn=32, E=8, k=2, capacity_factor=1.0,
                     gating="topk_softmax", act="swiglu", dtype="f32", seed=22),
    "T96_E16_f32": W("T96_E16_f32", T=96, d=48, ffn=40, E=16, k=4, capacity_factor=0.0,
                     gating="softmax_topk_renorm", act="gelu", dtype="f32", seed=23),
    "T150_E12_bf16": W("T150_E12_bf16", T=150, d=80, ffn=56, E=12, k=2, capacity_factor=1.5,
                       gating="softmax_topk", act="swiglu", dtype="bf16", seed=24),
    "T90_E40_bf16": W("T90_E40_bf16", T=90, d=48, ffn=24, E=40, k=4, capacity_factor=0.0,
                      gating="topk_softmax", act="swiglu", dtype="bf16", ep_ranks=8, seed=25),
    "T70_E20_f32": W("T70_E20_f32", T=70, d=56, ffn=32, E=20, k=1, capacity_factor=2.0,
                     gating="softmax_topk", act="gelu", dtype="f32", ep_ranks=4, placement="round_robin",
                     seed=26),
    # bf16 backward on transposed weights (at least 2000 rows per weight set
    # times m / (1 + m)): SwiGLU with round-robin placement and d, ffn that
    # end inside a 64-wide transpose tile; GELU on one expert; and the shared
    # experts' table alone (the routed one stays below the threshold)
    "T6144_E4_rr_swiglu_wt": W("T6144_E4_rr_swiglu_wt", T=6144, d=136, ffn=264, E=4, k=2,
                               capacity_factor=0.0, gating="softmax_topk", act="swiglu", dtype="bf16",
                               ep_ranks=2, placement="round_robin", seed=27),
    "T4200_E1_gelu_wt": W("T4200_E1_gelu_wt", T=4200, d=72, ffn=40, E=1, k=1, capacity_factor=0.0,
                          gating="softmax_topk", act="gelu", dtype="bf16", seed=28),
    "T3200_E4_shared_wt": W("T3200_E4_shared_wt", T=3200, d=64, ffn=32, E=4, k=2, capacity_factor=0.0,
                            gating="topk_softmax", act="swiglu", dtype="bf16", n_shared=1, ffn_shared=48,
                            seed=29),
    # weight-gradient launches with few tiles and long reductions split the
    # reduction into fp32 partials: the shared experts here (4 splits of
    # 1024 tokens) and the 2 routed experts of the next case (4 splits)
    "T4096_shared_splitk": W("T4096_shared_splitk", T=4096, d=64, ffn=32, E=8, k=2, capacity_factor=0.0,
                             gating="softmax_topk", act="swiglu", dtype="bf16", n_shared=2, ffn_shared=32,
                             seed=27),
    "T8192_E2_splitk": W("T8192_E2_splitk", T=8192, d=64, ffn=48, E=2, k=1, capacity_factor=0.0,
                         gating="softmax_topk", act="gelu", dtype="bf16", seed=28),
    # a strong router bias sends every token to experts 0 and 1 (counts 8192,
    # 8192, 0, 0) while the weight gradients split their reductions in 4: the
    # real items come first and the empty experts' zero partials after them
    # (with 4096 rows per expert on average, its dgrads run on transposed
    # weights, two of which no row reads; so do those of T8192_E2_splitk)
    "T8192_E4_skew_splitk": W("T8192_E4_skew_splitk", T=8192, d=64, ffn=48, E=4, k=2, capacity_factor=0.0,
                              gating="softmax_topk", act="swiglu", dtype="bf16", zipf_s=1.2, seed=43),
    # a skewed routing (the longest expert holds more than twice the mean
    # rows, one expert is empty) whose weight gradients split their reduction
    # in 2 and have 8 and 16 tiles per expert: each expert's tiles are spread
    # over the XCDs in runs, the empty expert's zeros come after them
    "T8192_E8_skew_runs": W("T8192_E8_skew_runs", T=8192, d=1024, ffn=512, E=8, k=2, capacity_factor=0.0,
                            gating="softmax_topk", act="swiglu", dtype="bf16", zipf_s=1.2, seed=51),
    # wide rows with a ragged tail: the bf16 route walks more than 32 K
    # blocks per wave (its chunked loop), the router-gradient and un-permute
    # launches end in a partial column block, and the GEMM reductions over d
    # end in a partial K step; the fp32 case does the same on the vector route
    "T96_d8200_bf16": W("T96_d8200_bf16", T=96, d=8200, ffn=48, E=4, k=2, capacity_factor=0.0,
                        gating="softmax_topk_renorm", act="gelu", dtype="bf16", seed=41),
    "T70_d4104_E20_f32": W("T70_d4104_E20_f32", T=70, d=4104, ffn=40, E=20, k=3, capacity_factor=1.2,
                           gating="softmax_topk", act="swiglu", dtype="f32", seed=42),
    # bf16 routing with 8 or 16 experts at model widths from 512 to 8192,
    # ragged T (down to a single token), the three gating modes and the
    # router bias; the last case spreads over several hundred workgroups
    "T333_d512_E8_dot2": W("T333_d512_E8_dot2", T=333, d=512, ffn=32, E=8, k=2, capacity_factor=1.0,
                           gating="topk_softmax", act="swiglu", dtype="bf16", seed=44),
    "T70_d1024_E8_dot2": W("T70_d1024_E8_dot2", T=70, d=1024, ffn=16, E=8, k=8, capacity_factor=0.0,
                           gating="softmax_topk", act="gelu", dtype="bf16", seed=45),
    "T1000_d2048_E16_dot2": W("T1000_d2048_E16_dot2", T=1000, d=2048, ffn=24, E=16, k=3, capacity_factor=0.0,
                              gating="softmax_topk_renorm", act="gelu", dtype="bf16", zipf_s=1.2, seed=46),
    "T257_d8192_E8_dot2": W("T257_d8192_E8_dot2", T=257, d=8192, ffn=16, E=8, k=1, capacity_factor=0.0,
                            gating="softmax_topk", act="gelu", dtype="bf16", seed=47),
    "T2500_d4096_E16_dot2": W("T2500_d4096_E16_dot2", T=2500, d=4096, ffn=16, E=16, k=2, capacity_factor=1.1,
                              gating="topk_softmax", act="swiglu", dtype="bf16", seed=48),
    "T1_d2048_E8_dot2": W("T1_d2048_E8_dot2", T=1, d=2048, ffn=16, E=8, k=2, capacity_factor=0.0,
                          gating="softmax_topk", act="gelu", dtype="bf16", seed=49),
    "T40000_d512_E8_dot2": W("T40000_d512_E8_dot2", T=40000, d=512, ffn=16, E=8, k=2, capacity_factor=1.0,
                             gating="softmax_topk_renorm", act="gelu", dtype="bf16", zipf_s=1.2, seed=50),
    # the balance loss (pages' coefficients 0.01 and 0.1) with its gradient
    # through dlogits, dW_r and dx: fp32, bf16 with 64 experts and shared
    # experts, and a skewed routing whose loss is well above coef
    "T777_E32_aux_f32": W("T777_E32_aux_f32", T=777, d=200, ffn=96, E=32, k=5, capacity_factor=1.3,
                          gating="topk_softmax", act="gelu", dtype="f32", aux_coef=0.1, seed=52),
    "T2000_E64_aux_shared": W("T2000_E64_aux_shared", T=2000, d=256, ffn=64, E=64, k=6, capacity_factor=0.0,
                              gating="softmax_topk", act="swiglu", dtype="bf16", ep_ranks=8, n_shared=2,
                              ffn_shared=32, aux_coef=0.01, seed=53),
    "T4096_E8_aux_skew": W("T4096_E8_aux_skew", T=4096, d=512, ffn=128, E=8, k=2, capacity_factor=1.0,
                           gating="softmax_topk_renorm", act="gelu", dtype="bf16", zipf_s=1.2, aux_coef=0.1,
                           seed=54),
    # more than 128 blocks of 256 tokens: dispatch takes its separate scan
    # launch instead of the per-workgroup sums of the block counts
    "T40000_E64_scan": W("T40000_E64_scan", T=40000, d=32, ffn=16, E=64, k=6, capacity_factor=1.0,
                         gating="softmax_topk", act="gelu", dtype="bf16", ep_ranks=8, seed=29),
}


# one token, d = 8, one expert: its single d_topk_w inner product cancels
# (about 700-fold on this seed), so it alone takes the fp32 dot-product floor
DOT_FLOOR_CASES = {"T1_E1_f32"}


@pytest.mark.parametrize("name", list(FUZZ))
def test_fuzz(name):
    announce(name)
    wl = FUZZ[name]
    inp = synth.make_inputs(wl)
    _, ref, errs = run_full_parity(wl, inp, dot_floor=name in DOT_FLOOR_CASES)
    print({k: f"{v:.2e}" for k, v in errs.items()}, "n =", ref["layout"]["n"], flush=True)
    if name == "T8192_E4_skew_splitk":  # the case is what its comment says
        assert list(np.asarray(ref["layout"]["kept_counts"])) == [8192, 8192, 0, 0]
    if name == "T4096_E8_aux_skew":  # skewed routing: the loss is well above its balanced value
        assert ref["aux_loss"] > 1.5 * wl.aux_coef
    if name == "T8192_E8_skew_runs":
        kept = np.asarray(ref["layout"]["kept_counts"])
        nz = int((kept > 0).sum())
        assert nz < wl.E and kept.max() * nz > 2 * kept.sum()


@pytest.mark.parametrize("name,wl", [
    ("ties_bf16_E8", W("ties_bf16_E8", T=700, d=64, ffn=32, E=8, k=2, capacity_factor=1.0,
                      gating="softmax_topk_renorm", act="gelu", dtype="bf16", seed=31)),
    # the same with wider rows on the bf16 MFMA route (8 and 16 experts)
    ("ties_bf16_E8_d512", W("ties_bf16_E8_d512", T=2000, d=512, ffn=16, E=8, k=2, capacity_factor=1.0,
                           gating="softmax_topk_renorm", act="gelu", dtype="bf16", seed=33)),
    ("ties_bf16_E16_d1024", W("ties_bf16_E16_d1024", T=1500, d=1024, ffn=16, E=16, k=3, capacity_factor=1.0,
                             gating="softmax_topk_renorm", act="gelu", dtype="bf16", seed=34)),
    ("ties_f32_E64", W("ties_f32_E64", T=300, d=32, ffn=16, E=64, k=6, capacity_factor=1.5,
                      gating="softmax_topk", act="swiglu", dtype="f32", ep_ranks=4, seed=32)),
])
def test_exact_ties(name, wl):
    """Dyadic inputs: every logit is exact in fp32, so the GPU logits equal
    the oracle's bit for bit and ties at the top-k boundary are frequent;
    routing must still match exactly (lower expert index wins)."""
    announce(name)
    inp = synth.make_inputs(wl, dyadic_router=True)
    layer, ref, _ = run_full_parity(wl, inp)
    np.testing.assert_array_equal(host(layer.logits), ref["logits_ref"])
    lg = ref["logits_ref"]
    s = np.sort(lg, axis=1)[:, ::-1]
    assert np.sum(s[:, wl.k - 1] == s[:, wl.k]) > 0, "the case must contain boundary ties"


def test_deterministic():
    """Two steps on the same inputs give bit-identical outputs."""
    announce("deterministic")
    wl = FUZZ["T1000_E64_rr_shared"]
    inp = synth.make_inputs(wl)
    layer, w, x, dy = make_layer(wl, inp)
    outs = []
    for _ in range(2):
        layer.step(x, dy, w)
        torch.cuda.synchronize()
        outs.append([bits(t).copy() for t in (layer.logits, layer.y, layer.dx, layer.dw1, layer.dw2,
                                               layer.dw_up, layer.dw_router, layer.dws_gate)]
                    + [host(layer.row_of).copy(), host(layer.topk_w).copy()])
    for a, b in zip(*outs):
        np.testing.assert_array_equal(a, b)


def test_route_on_dropped_tokens():
    """Capacity 1: almost every token is dropped; dropped tokens get y = 0
    and zero gate gradients."""
    announce("mostly_dropped")
    wl = W("mostly_dropped", T=500, d=64, ffn=32, E=4, k=1, capacity_factor=0.004,
           gating="softmax_topk", act="gelu", dtype="bf16", seed=40)
    inp = synth.make_inputs(wl)
    layer, ref, _ = run_full_parity(wl, inp)
    dropped = ref["layout"]["row_of"].reshape(wl.T, wl.k)[:, 0] < 0
    assert dropped.sum() >= wl.T - 4
    assert np.all(host(layer.y)[dropped] == 0.0)
    assert np.all(host(layer.d_topk_w)[dropped] == 0.0)


@pytest.mark.parametrize("name", ["T1000_E64_rr_shared", "T6144_E4_rr_swiglu_wt", "T3200_E4_shared_wt"])
def test_graph_replay(name):
    """The whole step captured in one HIP graph: three replays, each after
    eager work that overwrites every output, give outputs bit-identical to an
    eager step on the same inputs.  The last two workloads run the backward
    on transposed weights (routed, and shared experts)."""
    announce(f"graph_replay {name}")
    wl = FUZZ[name]
    inp = synth.make_inputs(wl)
    layer, w, x, dy = make_layer(wl, inp)
    outs = lambda: [t for t in (layer.logits, layer.y, layer.dx, layer.dw1, layer.dw2,  # noqa: E731
                                layer.dw_up, layer.dw_router, getattr(layer, "dws_gate", None),
                                getattr(layer, "dws_up", None), getattr(layer, "dws_down", None), layer.row_of,
                                layer.topk_w,
                                layer.x_perm, layer.expert_offsets) if t is not None]
    layer.step(x, dy, w)
    torch.cuda.synchronize()
    ref = [bits(t).copy() for t in outs()]
    graph = layer.capture_step(x, dy, w)
    for rep in range(3):
        for t in outs():
            t.fill_(-7 - rep)  # eager work between replays: every output scrambled
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for r, t in zip(ref, outs()):
            np.testing.assert_array_equal(bits(t), r)


def test_ffn_caller_group_table_of_65():
    """The grouped FFN through the C ABI with a caller-built table of 65
    groups, the most the ABI takes (weight set g for group g): one long
    group, many short ones and every fifth one empty.  The weight-gradient
    launches then read the group offsets in two chunks of 64 and, the table
    being skewed, spread the long group's tiles over the XCDs in runs; the
    empty groups' weight gradients must be exact zeros."""
    announce("ffn_caller_group_table_of_65")
    import oracle
    from mixture_experts_layer_36_amd import _native as nat, api

    G, d, F, rows_max = 65, 512, 512, 4096
    cfg = nat.make_config(2048, d, F, 64, 2, 0.0, "softmax_topk", "swiglu", "bf16")
    sizes = nat.plan(cfg)
    assert sizes.n_max == rows_max
    rng = np.random.default_rng(52)
    counts = rng.integers(1, 60, G)
    counts[0] = 1500
    counts[1::5] = 0
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    assert off[-1] <= rows_max and counts.max() * (counts > 0).sum() > 2 * counts.sum()

    x = synth.tensors.normal(61, (rows_max, d), "bf16")
    dy = synth.tensors.normal(62, (rows_max, d), "bf16")
    w_in = synth.tensors.normal(63, (G, d, F), "bf16", 0.05)
    w_up = synth.tensors.normal(64, (G, d, F), "bf16", 0.05)
    w_out = synth.tensors.normal(65, (G, F, d), "bf16", 0.05)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    bf = lambda *s: torch.zeros(*s, dtype=torch.bfloat16, device="cuda")
    xd, dyd, wi, wu, wo = dev(x), dev(dy), dev(w_in), dev(w_up), dev(w_out)
    act, h, y, dx = bf(rows_max, 2 * F), bf(rows_max, F), bf(rows_max, d), bf(rows_max, d)
    dwi, dwu, dwo = bf(G, d, F), bf(G, d, F), bf(G, F, d)
    ws = torch.empty(sizes.workspace_bytes, dtype=torch.uint8, device="cuda")
    offd = torch.from_numpy(off).cuda()
    grp = api.groups(G, F, rows_max, offd, use_placement=False)
    api.moe_expert_ffn_fwd(cfg, grp, xd, wi, wu, wo, act, h, y)
    api.moe_expert_ffn_bwd(cfg, grp, xd, wi, wu, wo, act, h, dyd, dx, dwi, dwu, dwo, ws)
    torch.cuda.synchronize()

    xf, dyf = oracle.to_f64(x), oracle.to_f64(dy)
    Wi, Wu, Wo = oracle.to_f64(w_in), oracle.to_f64(w_up), oracle.to_f64(w_out)
    n = int(off[-1])
    ref = {k: np.zeros(s) for k, s in (("d1", (n, F)), ("d2", (n, F)), ("h", (n, F)), ("y", (n, d)),
                                        ("dx", (n, d)), ("dwi", (G, d, F)), ("dwu", (G, d, F)),
                                        ("dwo", (G, F, d)))}
    for g in range(G):
        r0, r1 = int(off[g]), int(off[g + 1])
        fw = oracle.expert_ffn_forward(xf[r0:r1], Wi[g], Wo[g], "swiglu", Wu[g])
        bw = oracle.expert_ffn_backward(xf[r0:r1], dyf[r0:r1], Wi[g], Wo[g], "swiglu", Wu[g])
        fac = oracle.activation_factors(fw, "swiglu")
        ref["d1"][r0:r1], ref["d2"][r0:r1], ref["h"][r0:r1], ref["y"][r0:r1] = fac["d1"], fac["d2"], fw["h"], fw["o"]
        ref["dx"][r0:r1] = bw["dxp"]
        ref["dwi"][g], ref["dwu"][g], ref["dwo"][g] = bw["dw_in"], bw["dw_up"], bw["dw_out"]
    got_act = host(act)[:n]
    got = {"d1": got_act[:, :F], "d2": got_act[:, F:], "h": host(h)[:n], "y": host(y)[:n], "dx": host(dx)[:n],
           "dwi": host(dwi), "dwu": host(dwu), "dwo": host(dwo)}
    errs = {}
    for k in ref:
        e = float(np.max(np.abs(got[k] - ref[k])) / np.max(np.abs(ref[k])))
        errs[k] = e
        assert e <= TOL["bf16"], f"{k}: max|err|/max|ref| = {e:.3e}"
    empty = counts == 0
    for k in ("dwi", "dwu", "dwo"):
        assert np.all(got[k][empty] == 0.0), f"{k}: empty groups not exactly zero"
    print({k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
