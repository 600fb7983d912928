"""Pins of the oracle's expert FFN, combine and backward (CPU only).

Independent references used here:
  * a dense-masked evaluation: every expert on every token, then a 0/gate
    mask built by brute-force routing (no permutation, no row maps);
  * special cases: E = 1 is a dense FFN; k = E dropless is the soft mixture;
  * float64 central finite differences of <dy, y>;
  * torch CPU autograd on the same differentiable function;
  * closed values of GELU / SiLU and their derivatives.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def rand_layer(seed, T, d, F, E, act, n_shared=0, Fs=0, bias=False, scale=0.5):
    rng = np.random.default_rng(seed)
    p = dict(
        x=rng.normal(size=(T, d)),
        w_router=rng.normal(size=(d, E)) * scale,
        bias=rng.normal(size=E) if bias else None,
        w1=rng.normal(size=(E, d, F)) * 0.3,
        w_up=rng.normal(size=(E, d, F)) * 0.3 if act == "swiglu" else None,
        w2=rng.normal(size=(E, F, d)) * 0.3,
        dy=rng.normal(size=(T, d)),
        ws_gate=None, ws_up=None, ws_down=None,
    )
    if n_shared:
        p["ws_gate"] = rng.normal(size=(d, n_shared * Fs)) * 0.3
        p["ws_up"] = rng.normal(size=(d, n_shared * Fs)) * 0.3 if act == "swiglu" else None
        p["ws_down"] = rng.normal(size=(n_shared * Fs, d)) * 0.3
    return p


def run(p, **kw):
    return oracle.layer_forward_backward(
        p["x"], p["w_router"], p["bias"], p["w1"], p["w_up"], p["w2"], p["dy"],
        ws_gate=p["ws_gate"], ws_up=p["ws_up"], ws_down=p["ws_down"], **kw)


# ---------------------------------------------------------------- activations
def test_activation_values():
    assert oracle.gelu(np.array(0.0)) == 0.0
    assert oracle.gelu_grad(np.array(0.0)) == 0.5
    z = np.array([-3.0, -1.0, 0.5, 2.0, 8.0])
    ref = np.array([v * 0.5 * (1 + math.erf(v / math.sqrt(2))) for v in z])
    np.testing.assert_allclose(oracle.gelu(z), ref, rtol=1e-14)
    h = 1e-6
    np.testing.assert_allclose(oracle.gelu_grad(z),
                               (oracle.gelu(z + h) - oracle.gelu(z - h)) / (2 * h), rtol=1e-7, atol=1e-9)
    np.testing.assert_allclose(oracle.silu(np.array([0.0, 1.0])), [0.0, 1 / (1 + math.exp(-1))])
    assert abs(oracle.gelu(np.array(10.0)) - 10.0) < 1e-12


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
def test_activation_factors(act):
    """The factors a forward may save for the backward are the elementwise
    partial derivatives of h: torch CPU autograd of the same activation, and
    central differences of the oracle's forward in its pre-activations
    (x = I, so z = W1, a = W_gate, b = W_up; h is elementwise in them, so one
    shift of every entry gives every derivative)."""
    rng = np.random.default_rng(5)
    n, F = 6, 7
    w_in = rng.normal(size=(n, F)) * 2.0
    w_up = rng.normal(size=(n, F)) * 2.0 if act == "swiglu" else None
    w_out, eye = np.eye(F), np.eye(n)
    f = oracle.activation_factors(oracle.expert_ffn_forward(eye, w_in, w_out, act, w_up), act)
    a = torch.tensor(w_in, requires_grad=True)
    if act == "gelu":
        torch.nn.functional.gelu(a).sum().backward()
        np.testing.assert_allclose(f["d"], a.grad.numpy(), rtol=1e-12, atol=1e-14)
    else:
        b = torch.tensor(w_up, requires_grad=True)
        (torch.nn.functional.silu(a) * b).sum().backward()
        np.testing.assert_allclose(f["d1"], a.grad.numpy(), rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(f["d2"], b.grad.numpy(), rtol=1e-12, atol=1e-14)

    def h_at(wi, wu):
        return oracle.expert_ffn_forward(eye, wi, w_out, act, wu)["h"]
    eps = 1e-6
    fd = (h_at(w_in + eps, w_up) - h_at(w_in - eps, w_up)) / (2 * eps)
    np.testing.assert_allclose(f["d"] if act == "gelu" else f["d1"], fd, rtol=1e-6, atol=1e-8)
    if act == "swiglu":
        fd = (h_at(w_in, w_up + eps) - h_at(w_in, w_up - eps)) / (2 * eps)
        np.testing.assert_allclose(f["d2"], fd, rtol=1e-6, atol=1e-8)


# ---------------------------------------------------------------- dense references
def brute_route(lg, k, C):
    """Top-k by subset enumeration + sequential capacity counters ->
    mask M[t, e] in {0, 1}."""
    import itertools
    T, E = lg.shape
    M = np.zeros((T, E))
    chosen = []
    for t in range(T):
        best = None
        for sub in itertools.combinations(range(E), k):
            s = sum(lg[t, i] for i in sub)
            if best is None or s > best[0] or (s == best[0] and sub < best[1]):
                best = (s, sub)
        chosen.append(sorted(best[1], key=lambda i: (-lg[t, i], i)))
    cnt = [0] * E
    for t in range(T):
        for e in chosen[t]:
            if cnt[e] < C:
                M[t, e] = 1
            cnt[e] += 1
    return chosen, M


def dense_ffn(x, w_in, w_out, act, w_up=None):
    z = x @ w_in
    if act == "gelu":
        h = z * 0.5 * (1 + np.vectorize(math.erf)(z / math.sqrt(2)))
    else:
        h = z / (1 + np.exp(-z)) * (x @ w_up)
    return h @ w_out


def gates_dense(lg, chosen, gating):
    T, E = lg.shape
    G = np.zeros((T, E))
    for t in range(T):
        ex = np.exp(lg[t] - lg[t].max())
        p = ex / ex.sum()
        sel = chosen[t]
        for e in sel:
            if gating == "softmax_topk":
                G[t, e] = p[e]
            else:
                G[t, e] = p[e] / sum(p[m] for m in sel)
    return G


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
@pytest.mark.parametrize("gating", ["softmax_topk", "softmax_topk_renorm", "topk_softmax"])
def test_dense_masked_reference(act, gating):
    T, d, F, E, k, cf = 24, 6, 5, 4, 2, 0.75
    p = rand_layer(1, T, d, F, E, act, n_shared=2 if act == "swiglu" else 0, Fs=3, bias=True)
    out = run(p, k=k, gating=gating, act=act, capacity_factor=cf,
              n_shared=2 if act == "swiglu" else 0, backward=False)
    lg = p["x"] @ p["w_router"] + p["bias"]
    C = math.ceil(cf * k * T / E)
    chosen, M = brute_route(lg, k, C)
    G = gates_dense(lg, chosen, gating) * M
    y = np.zeros((T, d))
    for e in range(E):
        y += G[:, e:e + 1] * dense_ffn(p["x"], p["w1"][e], p["w2"][e], act,
                                       None if p["w_up"] is None else p["w_up"][e])
    if act == "swiglu":
        for s in range(2):
            c = slice(3 * s, 3 * s + 3)
            y += dense_ffn(p["x"], p["ws_gate"][:, c], p["ws_down"][c], act, p["ws_up"][:, c])
    assert M.sum() < T * k          # some drops happened
    np.testing.assert_allclose(out["y"], y, rtol=1e-12, atol=1e-12)


def test_single_expert_is_dense_ffn():
    T, d, F = 17, 5, 7
    p = rand_layer(2, T, d, F, 1, "gelu")
    out = run(p, k=1, gating="softmax_topk", act="gelu", capacity_factor=1.0, backward=False)
    np.testing.assert_allclose(out["topk_w"], 1.0)
    np.testing.assert_allclose(out["y"], dense_ffn(p["x"], p["w1"][0], p["w2"][0], "gelu"),
                               rtol=1e-12, atol=1e-13)


def test_k_equals_E_is_soft_mixture():
    T, d, F, E = 13, 4, 6, 3
    p = rand_layer(3, T, d, F, E, "swiglu")
    out = run(p, k=E, gating="softmax_topk", act="swiglu", capacity_factor=0.0, backward=False)
    lg = p["x"] @ p["w_router"]
    P = np.exp(lg - lg.max(1, keepdims=True))
    P /= P.sum(1, keepdims=True)
    y = sum(P[:, e:e + 1] * dense_ffn(p["x"], p["w1"][e], p["w2"][e], "swiglu", p["w_up"][e])
            for e in range(E))
    np.testing.assert_allclose(out["y"], y, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- gradients
def _routing_margin(lg, k):
    s = np.sort(lg, axis=1)[:, ::-1]
    if k >= lg.shape[1]:
        return np.inf
    return float(np.min(s[:, k - 1] - s[:, k]))


PARAMS = ["x", "w_router", "w1", "w_up", "w2", "ws_gate", "ws_up", "ws_down"]
GRADS = {"x": "dx", "w_router": "dw_router", "w1": "dw1", "w_up": "dw_up", "w2": "dw2",
         "ws_gate": "dws_gate", "ws_up": "dws_up", "ws_down": "dws_down"}


@pytest.mark.parametrize("act,gating,n_shared", [
    ("gelu", "softmax_topk", 0), ("gelu", "softmax_topk_renorm", 0),
    ("swiglu", "topk_softmax", 0), ("swiglu", "softmax_topk", 2)])
def test_finite_differences(act, gating, n_shared):
    T, d, F, E, k, cf = 20, 5, 4, 4, 2, 0.8
    p = None
    for seed in range(50):
        cand = rand_layer(10 + seed, T, d, F, E, act, n_shared=n_shared, Fs=3, bias=True)
        lg = cand["x"] @ cand["w_router"] + cand["bias"]
        if _routing_margin(lg, k) > 1e-3:
            p = cand
            break
    assert p is not None
    kw = dict(k=k, gating=gating, act=act, capacity_factor=cf, n_shared=n_shared)
    out = run(p, **kw)
    assert out["layout"]["n"] < T * k     # drops included
    rng = np.random.default_rng(0)
    h = 1e-6
    for name in PARAMS:
        if p[name] is None:
            continue
        v = rng.normal(size=p[name].shape)
        def loss(delta):
            q = dict(p)
            q[name] = p[name] + delta * v
            o = run(q, backward=False, **kw)
            # routing must not move under the perturbation
            assert np.array_equal(o["topk_idx"], out["topk_idx"])
            return float(np.sum(p["dy"] * o["y"]))
        fd = (loss(h) - loss(-h)) / (2 * h)
        an = float(np.sum(out[GRADS[name]] * v))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


def test_dlogits_sum_to_zero_and_support():
    p = rand_layer(5, 30, 6, 4, 8, "gelu", bias=False, scale=1.0)
    for gating in ("softmax_topk", "softmax_topk_renorm", "topk_softmax"):
        out = run(p, k=3, gating=gating, act="gelu", capacity_factor=0.9)
        dl = out["dlogits"]
        np.testing.assert_allclose(dl.sum(1), 0.0, atol=1e-13)
        if gating != "softmax_topk":
            mask = np.zeros_like(dl, dtype=bool)
            mask[np.arange(30)[:, None], out["topk_idx"]] = True
            assert np.all(dl[~mask] == 0.0)


def test_empty_expert_gradients_are_exact_zero():
    p = rand_layer(6, 16, 4, 3, 4, "swiglu")
    p["w_router"][:, 3] = 0.0
    p["bias"] = np.array([0.0, 0.0, 0.0, -100.0])
    out = run(p, k=2, gating="topk_softmax", act="swiglu", capacity_factor=0.0)
    assert out["layout"]["kept_counts"][3] == 0
    for key in ("dw1", "dw2", "dw_up"):
        assert np.all(out[key][3] == 0.0)


@pytest.mark.parametrize("act,gating", [("gelu", "softmax_topk_renorm"), ("swiglu", "softmax_topk")])
def test_torch_autograd_crosscheck(act, gating):
    T, d, F, E, k, cf = 32, 8, 6, 4, 2, 0.9
    p = rand_layer(7, T, d, F, E, act, n_shared=2, Fs=3, bias=True)
    out = run(p, k=k, gating=gating, act=act, capacity_factor=cf, n_shared=2)
    tt = {n: torch.tensor(v, dtype=torch.float64, requires_grad=True)
          for n, v in p.items() if v is not None and n not in ("dy", "bias")}
    bias = torch.tensor(p["bias"])
    lg = tt["x"] @ tt["w_router"] + bias
    idx = torch.tensor(out["topk_idx"])
    kept = torch.tensor(out["layout"]["row_of"].reshape(T, k) >= 0)
    P = torch.softmax(lg, dim=1)
    sel = torch.gather(P, 1, idx)
    g = sel if gating == "softmax_topk" else sel / sel.sum(1, keepdim=True)

    def ffn(xx, a_w, o_w, u_w=None):
        z = xx @ a_w
        if act == "gelu":
            hh = torch.nn.functional.gelu(z)
        else:
            hh = torch.nn.functional.silu(z) * (xx @ u_w)
        return hh @ o_w

    y = torch.zeros(T, d, dtype=torch.float64)
    for j in range(k):
        for e in range(E):
            m = (idx[:, j] == e) & kept[:, j]
            if m.any():
                ye = ffn(tt["x"][m], tt["w1"][e], tt["w2"][e],
                         tt["w_up"][e] if act == "swiglu" else None)
                y = y.index_add(0, torch.nonzero(m)[:, 0], g[m, j:j + 1] * ye)
    for s in range(2):
        c = slice(3 * s, 3 * s + 3)
        y = y + ffn(tt["x"], tt["ws_gate"][:, c], tt["ws_down"][c],
                    tt["ws_up"][:, c] if act == "swiglu" else None)
    np.testing.assert_allclose(y.detach().numpy(), out["y"], rtol=1e-12, atol=1e-12)
    (y * torch.tensor(p["dy"])).sum().backward()
    for name, t in tt.items():
        np.testing.assert_allclose(t.grad.numpy(), out[GRADS[name]], rtol=1e-10, atol=1e-11,
                                   err_msg=name)
