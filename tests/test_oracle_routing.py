"""Pins of the oracle's routing, capacity and dispatch layout (CPU only).

Each check is independent of the oracle's own code path: brute-force subset
enumeration, a literal sequential simulation with per-expert counters,
closed forms, and the tutorial's worked all-to-all example.
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def dyadic_logits(rng, T, E, levels=4):
    """Logits on a coarse grid so that equal values (ties) are frequent."""
    return rng.integers(-levels, levels + 1, size=(T, E)).astype(np.float64) / 4.0


# ---------------------------------------------------------------- top-k
def brute_topk(row, k):
    """Max-sum k-subset, ties -> lexicographically smallest sorted index
    tuple; then ordered by (value desc, index asc)."""
    E = len(row)
    best = None
    for sub in itertools.combinations(range(E), k):
        s = sum(row[i] for i in sub)
        if best is None or s > best[0] or (s == best[0] and sub < best[1]):
            best = (s, sub)
    return sorted(best[1], key=lambda i: (-row[i], i))


@pytest.mark.parametrize("seed", range(6))
def test_topk_matches_bruteforce(seed):
    rng = np.random.default_rng(seed)
    for E in (1, 2, 3, 5, 8):
        for k in range(1, min(E, 3) + 1):
            lg = dyadic_logits(rng, 40, E, levels=2)
            got = oracle.select_topk(lg, k)
            for t in range(lg.shape[0]):
                assert list(got[t]) == brute_topk(list(lg[t]), k), (E, k, t)


def test_topk_signed_zero_and_ties():
    lg = np.array([[0.0, -0.0, 0.0, -1.0], [-0.0, 0.0, 1.0, 1.0]])
    got = oracle.select_topk(lg, 3)
    assert got.tolist() == [[0, 1, 2], [2, 3, 0]]


def test_topk_rejects_nonfinite():
    with pytest.raises(ValueError):
        oracle.select_topk(np.array([[0.0, np.nan]]), 1)


# ---------------------------------------------------------------- gates
@pytest.mark.parametrize("seed", range(3))
def test_gate_weight_identities(seed):
    rng = np.random.default_rng(seed)
    lg = rng.normal(size=(50, 8)) * 3
    idx = oracle.select_topk(lg, 3)
    p_full = np.exp(lg) / np.exp(lg).sum(1, keepdims=True)
    g0 = oracle.gate_weights(lg, idx, "softmax_topk")
    np.testing.assert_allclose(g0, np.take_along_axis(p_full, idx, 1), rtol=1e-13)
    g1 = oracle.gate_weights(lg, idx, "softmax_topk_renorm")
    g2 = oracle.gate_weights(lg, idx, "topk_softmax")
    np.testing.assert_allclose(g1.sum(1), 1.0, rtol=1e-13)
    np.testing.assert_allclose(g1, g2, rtol=1e-12)
    # weights follow the selection order
    assert np.all(np.diff(g0, axis=1) <= 0)
    idx1 = oracle.select_topk(lg, 1)
    np.testing.assert_allclose(oracle.gate_weights(lg, idx1, "softmax_topk_renorm"), 1.0)


def test_softmax_shift_invariance_large_logits():
    lg = np.array([[1000.0, 999.0, -1000.0]])
    idx = oracle.select_topk(lg, 2)
    g = oracle.gate_weights(lg, idx, "softmax_topk")
    np.testing.assert_allclose(g[0], [1 / (1 + np.exp(-1)), np.exp(-1) / (1 + np.exp(-1))])


# ---------------------------------------------------------------- capacity
def test_capacity_of_the_workloads():
    assert oracle.capacity(512, 4, 1, 1.25) == 160
    assert oracle.capacity(8192, 8, 2, 1.25) == 2560
    assert oracle.capacity(16384, 16, 2, 1.0) == 2048
    assert oracle.capacity(16384, 8, 2, 0.0) == 16384
    assert oracle.capacity(100, 2, 2, 5.0) == 100        # capped at T
    assert oracle.capacity(10, 3, 1, 1.0) == 4           # ceil(10/3)
    assert oracle.capacity(7, 64, 1, 0.01) == 1          # ceil of a tiny value


# ---------------------------------------------------------------- layout
def sequential_dispatch(idx, E, C, R, placement):
    """Literal simulation: tokens arrive in order; each expert has a counter
    and accepts while the counter is below C.  Buffers are then laid out
    rank by rank, local expert by local expert."""
    T, k = idx.shape
    counters = [0] * E
    accepted = [[] for _ in range(E)]        # (t, j) in arrival order
    pos = np.zeros((T, k), dtype=np.int64)
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j])
            pos[t, j] = counters[e]
            if counters[e] < C:
                accepted[e].append((t, j))
            counters[e] += 1
    L = E // R
    if placement == "contiguous":
        on_rank = [[q * L + l for l in range(L)] for q in range(R)]
    else:
        on_rank = [[q + R * l for l in range(L)] for q in range(R)]
    rows = []
    send_counts = []
    seg_experts = []
    for q in range(R):
        c = 0
        for e in on_rank[q]:
            rows.extend(accepted[e])
            c += len(accepted[e])
            seg_experts.append(e)
        send_counts.append(c)
    row_of = -np.ones((T, k), dtype=np.int64)
    for r, (t, j) in enumerate(rows):
        row_of[t, j] = r
    return dict(pos=pos, counters=counters, rows=rows, row_of=row_of,
                send_counts=send_counts, slot_expert=seg_experts,
                accepted=accepted)


@pytest.mark.parametrize("seed", range(8))
@pytest.mark.parametrize("placement", ["contiguous", "round_robin"])
def test_layout_matches_sequential_simulation(seed, placement):
    rng = np.random.default_rng(100 + seed)
    T = int(rng.integers(1, 80))
    E = int(rng.choice([1, 2, 4, 6, 8, 12]))
    R = int(rng.choice([r for r in (1, 2, 3, 4) if E % r == 0]))
    k = int(rng.integers(1, min(E, 4) + 1))
    C = int(rng.integers(0, T + 2))
    lg = dyadic_logits(rng, T, E)
    # skew towards low experts so that drops happen
    lg -= np.arange(E)[None, :] * 0.25
    idx = oracle.select_topk(lg, k)
    lay = oracle.dispatch_layout(idx, E, C, R, placement)
    ref = sequential_dispatch(idx, E, C, R, placement)
    np.testing.assert_array_equal(lay["pos"], ref["pos"])
    np.testing.assert_array_equal(lay["row_of"], ref["row_of"].reshape(lay["row_of"].shape))
    np.testing.assert_array_equal(lay["raw_counts"], ref["counters"])
    np.testing.assert_array_equal(lay["send_counts"], ref["send_counts"])
    np.testing.assert_array_equal(lay["slot_expert"], ref["slot_expert"])
    assert lay["n"] == len(ref["rows"])
    assert [tuple(divmod(int(a), k)) for a in lay["assign_of_row"]] == ref["rows"]


@pytest.mark.parametrize("seed", range(6))
def test_layout_invariants(seed):
    rng = np.random.default_rng(200 + seed)
    T, E, k = 64, 8, 3
    C = int(rng.integers(0, 30))
    lg = rng.normal(size=(T, E)) - np.arange(E)[None, :] * 0.3
    idx = oracle.select_topk(lg, k)
    lay = oracle.dispatch_layout(idx, E, C)
    kept = lay["kept_counts"]
    off = lay["expert_offsets"]
    assert np.all(kept <= C)
    assert lay["n"] == kept.sum() == off[-1]
    a = lay["assign_of_row"]
    assert len(np.unique(a)) == len(a)                  # each kept (t,j) once
    for e in range(E):
        rows = a[off[e]:off[e + 1]]
        toks = rows // k
        assert np.all(idx[toks, rows % k] == e)         # right expert
        assert np.all(np.diff(toks) > 0)                # ascending tokens
        dropped = [t for t in range(T) if e in idx[t] and t not in set(toks)]
        if dropped:
            assert kept[e] == C
            assert len(toks) == 0 or toks.max() < min(dropped)
    # every (t, j) is either kept exactly once or marked dropped
    ro = lay["row_of"]
    assert np.all((ro == -1) | ((ro >= 0) & (ro < lay["n"])))
    assert np.sum(ro >= 0) == lay["n"]


def test_dropless_and_zero_capacity():
    rng = np.random.default_rng(7)
    idx = oracle.select_topk(rng.normal(size=(33, 5)), 2)
    lay = oracle.dispatch_layout(idx, 5, 33)
    assert lay["n"] == 66 and np.all(lay["row_of"] >= 0)
    lay0 = oracle.dispatch_layout(idx, 5, 0)
    assert lay0["n"] == 0 and np.all(lay0["row_of"] == -1)


def test_zero_router_closed_form():
    """W_r = 0 and no bias: all logits tie, so every token picks experts
    0..k-1; raw_e = T for e < k; tokens t < C are kept; gates are 1/E
    (softmax_topk) or 1/k (renormalised)."""
    T, d, E, k, cf = 40, 8, 6, 3, 0.5
    x = np.random.default_rng(0).normal(size=(T, d))
    lg = oracle.gate_logits(x, np.zeros((d, E)))
    idx = oracle.select_topk(lg, k)
    assert np.all(idx == np.arange(k)[None, :])
    C = oracle.capacity(T, E, k, cf)
    assert C == 10
    lay = oracle.dispatch_layout(idx, E, C)
    np.testing.assert_array_equal(lay["raw_counts"], [T] * k + [0] * (E - k))
    np.testing.assert_array_equal(lay["kept_counts"], [C] * k + [0] * (E - k))
    kept_tokens = np.nonzero(lay["row_of"][:, 0] >= 0)[0]
    np.testing.assert_array_equal(kept_tokens, np.arange(C))
    np.testing.assert_allclose(oracle.gate_weights(lg, idx, "softmax_topk"), 1.0 / E)
    np.testing.assert_allclose(oracle.gate_weights(lg, idx, "softmax_topk_renorm"), 1.0 / k)


# ---------------------------------------------------------------- pages' examples
def test_placement_example():
    """8 experts on 4 devices: Dev0 holds E0, E1 and E2 lives on Dev1
    (tutorial ch.4, 专家并行 三, 图示说明)."""
    assert [oracle.expert_rank(e, 8, 4, "contiguous") for e in range(8)] == [0, 0, 1, 1, 2, 2, 3, 3]
    assert oracle.expert_rank(2, 8, 4, "contiguous") == 1
    # EP sizing examples of the practice section: 64 experts over EP=2 -> 32
    # per GPU, over EP=8 -> 8 per GPU.
    for R, per in ((2, 32), (8, 8)):
        ranks = [oracle.expert_rank(e, 64, R, "contiguous") for e in range(64)]
        assert all(ranks.count(q) == per for q in range(R))


def test_alltoall_worked_example():
    """The 4-device data-flow example of the all-to-all section, each
    device run as its own single-GPU layer, then a loopback exchange."""
    g = json.load(open(os.path.join(GOLDEN, "a2a_worked_example.json")))
    E = R = 4
    sends = []
    for dev, spec in enumerate(g["devices"]):
        dest = spec["dest_rank"]
        lg = np.zeros((3, E))
        lg[np.arange(3), dest] = 1.0
        idx = oracle.select_topk(lg, 1)
        lay = oracle.dispatch_layout(idx, E, oracle.capacity(3, E, 1, 0.0), R)
        assert lay["send_counts"].tolist() == g["expected_send_counts"][dev]
        segs = []
        for q in range(R):
            rows = lay["assign_of_row"][lay["send_offsets"][q]:lay["send_offsets"][q + 1]]
            segs.append([spec["tokens"][int(a)] for a in rows])
        assert segs == g["expected_segments"][dev]
        sends.append(segs)
    received = [sum((sends[i][q] for i in range(4)), []) for q in range(4)]
    assert received == g["expected_received"]
