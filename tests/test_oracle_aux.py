"""Pins of the oracle's balance loss (CPU only).

The loss follows a reading (the pages give its coefficient and its goal, not
its formula): L = coef * E * sum_e f_e P_e, f_e the share of routing choices
on expert e, P_e the mean router probability of e.  Pinned by what that
definition and the pages fix, independently of the oracle's code:
  * closed values: a zero router (every probability 1/E) and any routing
    that chooses every expert equally often give L = coef, the value the
    pages call ideal (near 0 for their coefficients 0.01 - 0.1); all choices
    on one expert with its probability near 1 give coef * E / k;
  * brute force: the same sum written as explicit loops over tokens,
    choices and experts;
  * its gradient against float64 central differences along random
    directions (routing held fixed), torch autograd, and softmax shift
    invariance (each token's gradient sums to 0);
  * the whole layer: <dy, y> + L differentiated by finite differences in x
    and W_r.
"""
import numpy as np
import pytest
import torch

import oracle


def test_zero_router_gives_coef():
    for T, E, k in [(10, 4, 1), (33, 8, 2), (7, 64, 6)]:
        lg = np.zeros((T, E))
        idx = oracle.select_topk(lg, k)
        assert np.array_equal(idx, np.tile(np.arange(k), (T, 1)))  # ties -> lowest indices
        for coef in (0.01, 0.1, 1.0):
            assert abs(oracle.balance_loss(lg, idx, E, coef) - coef) < 1e-15


def test_equal_choice_counts_give_coef_for_any_probabilities():
    rng = np.random.default_rng(3)
    T, E, k = 64, 8, 2
    # token t chooses experts 2t mod E and 2t+1 mod E: every expert exactly T k / E times
    idx = np.stack([(2 * np.arange(T)) % E, (2 * np.arange(T) + 1) % E], axis=1)
    assert np.all(np.bincount(idx.ravel(), minlength=E) == T * k // E)
    lg = rng.normal(size=(T, E)) * 3.0
    assert abs(oracle.balance_loss(lg, idx, E, 0.01) - 0.01) < 1e-15


def test_all_choices_on_one_expert():
    T, E, k = 50, 16, 1
    lg = np.zeros((T, E))
    lg[:, 5] = 60.0   # probability of expert 5 within 1e-25 of 1
    idx = oracle.select_topk(lg, k)
    assert np.all(idx == 5)
    np.testing.assert_allclose(oracle.balance_loss(lg, idx, E, 0.1), 0.1 * E / k, rtol=1e-12)


def test_matches_brute_force_loops():
    rng = np.random.default_rng(4)
    T, E, k, coef = 23, 7, 3, 0.05
    lg = rng.normal(size=(T, E))
    idx = oracle.select_topk(lg, k)
    f = [0.0] * E
    for t in range(T):
        for j in range(k):
            f[int(idx[t, j])] += 1.0 / (T * k)
    P = [0.0] * E
    for t in range(T):
        z = sum(np.exp(lg[t, m]) for m in range(E))
        for e in range(E):
            P[e] += np.exp(lg[t, e]) / z / T
    ref = coef * E * sum(f[e] * P[e] for e in range(E))
    assert abs(oracle.balance_loss(lg, idx, E, coef) - ref) < 1e-14


def test_gradient_finite_differences_autograd_and_shift_invariance():
    rng = np.random.default_rng(5)
    T, E, k, coef = 17, 6, 2, 0.1
    lg = rng.normal(size=(T, E))
    idx = oracle.select_topk(lg, k)
    g = oracle.balance_loss_grad(lg, idx, E, coef)
    np.testing.assert_allclose(g.sum(axis=1), 0.0, atol=1e-16)
    h = 1e-6
    for _ in range(5):
        v = rng.normal(size=lg.shape)
        assert np.array_equal(oracle.select_topk(lg + h * v, k), idx)
        fd = (oracle.balance_loss(lg + h * v, idx, E, coef) - oracle.balance_loss(lg - h * v, idx, E, coef)) / (2 * h)
        assert abs(fd - np.sum(g * v)) <= 1e-9
    lt = torch.tensor(lg, requires_grad=True)
    f = torch.tensor(np.bincount(idx.ravel(), minlength=E) / (T * k))
    L = coef * E * (f * torch.softmax(lt, dim=1).mean(dim=0)).sum()
    L.backward()
    np.testing.assert_allclose(lt.grad.numpy(), g, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("gating", ["softmax_topk", "topk_softmax"])
def test_layer_gradient_includes_the_balance_loss(gating):
    """Finite differences of <dy, y> + L in x and W_r: the layer's dx and
    dW_r carry the balance loss through dlogits."""
    rng = np.random.default_rng(9)
    T, d, F, E, k, coef = 24, 5, 4, 4, 2, 0.3
    for _ in range(100):
        x = rng.normal(size=(T, d))
        wr = rng.normal(size=(d, E)) * 0.7
        s = np.sort(x @ wr, axis=1)[:, ::-1]
        if np.min(s[:, k - 1] - s[:, k]) > 1e-3:
            break
    w1 = rng.normal(size=(E, d, F)) * 0.3
    w2 = rng.normal(size=(E, F, d)) * 0.3
    dy = rng.normal(size=(T, d))
    kw = dict(k=k, gating=gating, act="gelu", capacity_factor=0.0, aux_coef=coef)
    out = oracle.layer_forward_backward(x, wr, None, w1, None, w2, dy, **kw)
    base = oracle.layer_forward_backward(x, wr, None, w1, None, w2, dy, **{**kw, "aux_coef": 0.0})
    assert out["aux_loss"] > 0 and not np.allclose(out["dw_router"], base["dw_router"])

    def objective(xx, ww):
        o = oracle.layer_forward_backward(xx, ww, None, w1, None, w2, dy, backward=False, **kw)
        assert np.array_equal(o["topk_idx"], out["topk_idx"])
        return float(np.sum(dy * o["y"]) + o["aux_loss"])

    h = 1e-6
    for name, grad in (("x", out["dx"]), ("w_router", out["dw_router"])):
        v = rng.normal(size=x.shape if name == "x" else wr.shape)
        if name == "x":
            fd = (objective(x + h * v, wr) - objective(x - h * v, wr)) / (2 * h)
        else:
            fd = (objective(x, wr + h * v) - objective(x, wr - h * v)) / (2 * h)
        assert abs(fd - np.sum(grad * v)) <= 1e-6 * max(1.0, abs(fd)), name
