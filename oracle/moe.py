"""Float64 numpy oracle of one GPU's share of the MoE layer, forward and backward.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Page references (titles as printed on the pages):
  [EP]    tutorial ch.4 "扩展 MoE 模型——迈向分布式训练", section
          "专家并行：在不同设备上分配专家" (二 the four-step EP flow;
          三 the 4-device / 8-expert picture; 五 expert placement).
  [EPDP]  same page, section "专家并行与数据并行的结合", 三 training flow
          (forward, backward: gradients routed back to the experts, expert
          parameter gradients computed locally; router gradients aggregated).
  [A2A]   same page, section "All-to-All 通信模式", 二 mechanism (send sets
          S_ik), 三 the 4-device data-flow example, 六 variable-size
          exchanges (Alltoallv, grouped sends).
  [PP]    same page, "MoE 模型的流水线并行", 三 (gate, route, experts,
          outputs merged).
  [FW]    same page, "用于分布式 MoE 的主流框架与库": Tutel's top-k gate
          (k=2) and ffn experts; DeepSpeed's moe block.
  [PIPER] Piper summary, 方法论 1 (resource model: routing table, expert
          capacity as a model input).
  [FSMOE] FSMoE abstract: token routing, token communication, expert
          computation, expert parallelism as the four MoE modules.

Readings adopted where the pages are silent:
  * capacity C = ceil(cf*k*T/E) in double from the fp32 factor, capped at T;
    cf <= 0 means dropless (C = T);
  * overflow is dropped in token order: an expert keeps the C lowest-index
    tokens that chose it;
  * selection key is the fp32 logit (bias included), larger first, equal
    values -> lower expert index;
  * gate weights per mode as in gate_weights(); dropped assignments
    contribute nothing and weights are not renormalised after drops;
  * GELU is the exact erf form; SwiGLU is silu(x Wg) * (x Wu) then W_down;
    no biases in the experts;
  * shared experts have weight 1 and see every token;
  * expert placement over EP ranks is contiguous by default (the 4-device
    picture puts E2 on Dev1), round-robin selectable; within a rank the
    segments go by local expert, then by token.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import erf

GATINGS = ("softmax_topk", "softmax_topk_renorm", "topk_softmax")
ACTS = ("gelu", "swiglu")
PLACEMENTS = ("contiguous", "round_robin")


# --------------------------------------------------------------------------
# storage conversions (bf16 bit patterns / fp32 -> float64)
# --------------------------------------------------------------------------
def to_f64(a: np.ndarray) -> np.ndarray:
    """Widen an fp32 array, or bf16 stored as uint16 bit patterns, to float64."""
    if a is None:
        return None
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


# --------------------------------------------------------------------------
# routing  [EP 二 step 1, A2A 二: the replicated gate g(x); FW: top-k gate]
# --------------------------------------------------------------------------
def gate_logits(x: np.ndarray, w_router: np.ndarray, bias=None) -> np.ndarray:
    """l[t, e] = sum_i x[t, i] * W_r[i, e] + b[e]  ([EP] 二 step 1, the
    replicated router scores each local token against every expert)."""
    l = x @ w_router
    if bias is not None:
        l = l + np.asarray(bias, dtype=np.float64)[None, :]
    return l


def select_topk(logits: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k experts of each token ([FW] top-k gate, k chosen
    experts per token), ordered by (logit descending, expert index
    ascending): a stable sort of the negated logits keeps equal values in
    index order.  Inputs must be finite."""
    logits = np.asarray(logits, dtype=np.float64)
    if not np.all(np.isfinite(logits)):
        raise ValueError("logits must be finite")
    order = np.argsort(-logits, axis=1, kind="stable")
    return order[:, :k].astype(np.int64)


def softmax(l: np.ndarray, axis: int = -1) -> np.ndarray:
    m = np.max(l, axis=axis, keepdims=True)
    e = np.exp(l - m)
    return e / np.sum(e, axis=axis, keepdims=True)


def gate_weights(logits: np.ndarray, idx: np.ndarray, gating: str) -> np.ndarray:
    """Gate weight g[t, j] of the j-th chosen expert ([A2A] 二, the gate g(x)).

    softmax_topk        g_j = softmax(l)[e_j]
    softmax_topk_renorm g_j = softmax(l)[e_j] / sum_m softmax(l)[e_m]
    topk_softmax        g_j = exp(l[e_j]) / sum_m exp(l[e_m])  (m over chosen)
    """
    if gating not in GATINGS:
        raise ValueError(gating)
    p = softmax(logits, axis=1)
    sel = np.take_along_axis(p, idx, axis=1)
    if gating == "softmax_topk":
        return sel
    if gating == "softmax_topk_renorm":
        return sel / np.sum(sel, axis=1, keepdims=True)
    return softmax(np.take_along_axis(logits, idx, axis=1), axis=1)


# --------------------------------------------------------------------------
# capacity, positions, layout  [PIPER 方法论 1; A2A 二/六; EP 三/五]
# --------------------------------------------------------------------------
def capacity(T: int, E: int, k: int, capacity_factor: float) -> int:
    """Expert capacity ([PIPER] 方法论 1 names it as a model input).
    C = ceil(cf * k * T / E), evaluated left to right in double from the
    fp32 factor and capped at T; cf <= 0 gives the dropless C = T."""
    cf = float(np.float32(capacity_factor))
    if cf <= 0.0:
        return int(T)
    return int(min(T, math.ceil(cf * k * T / E)))


def expert_rank(e: int, E: int, R: int, placement: str) -> int:
    """EP rank holding expert e ([EP] 一: N experts spread over D devices,
    N/D each; 三: contiguous picture; 五: round-robin is common)."""
    L = E // R
    return e // L if placement == "contiguous" else e % R


def expert_local(e: int, E: int, R: int, placement: str) -> int:
    L = E // R
    return e % L if placement == "contiguous" else e // R


def slot_order(E: int, R: int, placement: str) -> np.ndarray:
    """Experts listed in send-buffer order: by rank, then by local index."""
    if placement not in PLACEMENTS or R < 1 or E % R:
        raise ValueError("bad placement")
    keys = [(expert_rank(e, E, R, placement), expert_local(e, E, R, placement), e)
            for e in range(E)]
    return np.array([e for _, _, e in sorted(keys)], dtype=np.int64)


def assignment_positions(idx: np.ndarray, E: int) -> np.ndarray:
    """pos(t, j) = number of earlier tokens t' < t whose chosen set contains
    e_{t,j} (token-order arrival at the expert)."""
    T, k = idx.shape
    chose = np.zeros((T, E), dtype=np.int64)
    chose[np.arange(T)[:, None], idx] = 1
    earlier = np.cumsum(chose, axis=0) - chose
    return np.take_along_axis(earlier, idx, axis=1)


def dispatch_layout(idx: np.ndarray, E: int, C: int, R: int = 1,
                    placement: str = "contiguous") -> dict:
    """Counts, offsets, send layout and row maps of the dispatch.

    The per-expert buffers ([PIPER] 方法论 1 capacity) are laid out as the
    all-to-all send buffer: device i sends S_ik, its tokens whose expert
    lives on device k ([A2A] 二), so segment q holds the kept assignments of
    the experts on rank q, by local expert then token ([A2A] 六: variable
    sizes).  An assignment (t, j) is kept iff pos(t, j) < C.
    """
    T, k = idx.shape
    pos = assignment_positions(idx, E)
    kept_mask = pos < C
    raw = np.bincount(idx.ravel(), minlength=E).astype(np.int64)
    kept = np.minimum(raw, C)
    order = slot_order(E, R, placement)
    slot_offsets = np.zeros(E + 1, dtype=np.int64)
    slot_offsets[1:] = np.cumsum(kept[order])
    start = np.empty(E, dtype=np.int64)
    start[order] = slot_offsets[:-1]
    row = start[idx] + pos
    row_of = np.where(kept_mask, row, -1).astype(np.int64)
    n = int(slot_offsets[-1])
    assign_of_row = np.full(n, -1, dtype=np.int64)
    tt, jj = np.nonzero(kept_mask)
    assign_of_row[row[tt, jj]] = tt * k + jj
    L = E // R
    send_counts = np.array([slot_offsets[(q + 1) * L] - slot_offsets[q * L]
                            for q in range(R)], dtype=np.int64)
    send_offsets = np.zeros(R + 1, dtype=np.int64)
    send_offsets[1:] = np.cumsum(send_counts)
    return dict(pos=pos, kept_mask=kept_mask, raw_counts=raw,
                kept_counts=kept, slot_expert=order,
                expert_offsets=slot_offsets, expert_start=start,
                row_of=row_of, assign_of_row=assign_of_row, n=n,
                send_counts=send_counts, send_offsets=send_offsets)


def permute_rows(x: np.ndarray, layout: dict, k: int) -> np.ndarray:
    """x_perm[row(t, j)] = x[t] for every kept assignment ([EP] 二 step 2:
    tokens sent to the device of their expert; here written, not sent)."""
    n = layout["n"]
    xp = np.zeros((n, x.shape[1]), dtype=x.dtype)
    a = layout["assign_of_row"]
    xp[np.arange(n)] = x[a // k]
    return xp


# --------------------------------------------------------------------------
# expert FFN  [EP 二 step 3; FW: ffn experts]
# --------------------------------------------------------------------------
def gelu(z):
    """Exact GELU, z * Phi(z) = z/2 * (1 + erf(z / sqrt 2))."""
    return 0.5 * z * (1.0 + erf(z / math.sqrt(2.0)))


def gelu_grad(z):
    """d GELU / dz = Phi(z) + z * phi(z)."""
    return 0.5 * (1.0 + erf(z / math.sqrt(2.0))) + z * np.exp(-0.5 * z * z) / math.sqrt(2.0 * math.pi)


def sigmoid(a):
    return 1.0 / (1.0 + np.exp(-a))


def silu(a):
    return a * sigmoid(a)


def expert_ffn_forward(xp, w_in, w_out, act: str, w_up=None) -> dict:
    """One expert on its rows ([EP] 二 step 3: each device runs its local
    experts on the tokens it received; [FW] experts of type ffn).

    gelu:   z = xp W1;  h = GELU(z);              o = h W2
    swiglu: a = xp Wg;  b = xp Wu;  h = silu(a)*b; o = h W_down
    Any subset of rows, or of hidden units (columns of W_in / rows of W_out),
    may be passed: rows are independent and hidden units add up in o.
    """
    out = {}
    if act == "gelu":
        z = xp @ w_in
        h = gelu(z)
        out["z"] = z
    elif act == "swiglu":
        a = xp @ w_in
        b = xp @ w_up
        h = silu(a) * b
        out["a"] = a
        out["b"] = b
    else:
        raise ValueError(act)
    out["h"] = h
    out["o"] = h @ w_out
    return out


def expert_ffn_backward(xp, do, w_in, w_out, act: str, w_up=None) -> dict:
    """Gradients of one expert ([EPDP] 三.3: gradients routed back to the
    expert's device, expert parameter gradients computed locally).

    gelu:   dh = do W2^T; dz = dh * GELU'(z); dW2 = h^T do; dW1 = xp^T dz;
            dxp = dz W1^T
    swiglu: dh = do Wd^T; s = sigmoid(a); da = dh * b * s * (1 + a (1 - s));
            db = dh * silu(a); dWd = h^T do; dWg = xp^T da; dWu = xp^T db;
            dxp = da Wg^T + db Wu^T
    With no rows, every weight gradient is exactly zero.
    """
    fwd = expert_ffn_forward(xp, w_in, w_out, act, w_up)
    h = fwd["h"]
    dh = do @ w_out.T
    out = {"dw_out": h.T @ do}
    if act == "gelu":
        dz = dh * gelu_grad(fwd["z"])
        out["dw_in"] = xp.T @ dz
        out["dxp"] = dz @ w_in.T
    else:
        a, b = fwd["a"], fwd["b"]
        s = sigmoid(a)
        da = dh * b * s * (1.0 + a * (1.0 - s))
        db = dh * silu(a)
        out["dw_in"] = xp.T @ da
        out["dw_up"] = xp.T @ db
        out["dxp"] = da @ w_in.T + db @ w_up.T
    return out


def activation_factors(fwd: dict, act: str) -> dict:
    """Partial derivatives of the activation h at a forward's
    pre-activations (the factors of the chain rule in [EPDP] 三.3 that take
    dL/dh to dL/dz, or to dL/da and dL/db):

    gelu:   d  = dh/dz = GELU'(z)
    swiglu: d1 = dh/da = b * s * (1 + a (1 - s)),  s = sigmoid(a)
            d2 = dh/db = silu(a)
    so that dz = dh * d, da = dh * d1, db = dh * d2 as in
    expert_ffn_backward.  A forward may keep these in place of z or a, b
    when h itself is saved.
    """
    if act == "gelu":
        return {"d": gelu_grad(fwd["z"])}
    if act == "swiglu":
        a, b = fwd["a"], fwd["b"]
        s = sigmoid(a)
        return {"d1": b * s * (1.0 + a * (1.0 - s)), "d2": silu(a)}
    raise ValueError(act)


# --------------------------------------------------------------------------
# combine  [EP 二 step 4; PP 三 outputs merged]
# --------------------------------------------------------------------------
def combine(o_perm, row_of, g, y_shared=None) -> np.ndarray:
    """y[t] = sum over kept j of g[t, j] * o[row(t, j)]  (+ shared experts).

    ([EP] 二 step 4: results return to the token's device in sequence
    order; [PP] 三: outputs merged.)  Dropped assignments contribute 0."""
    T, k = row_of.shape
    y = np.zeros((T, o_perm.shape[1]), dtype=np.float64)
    for j in range(k):
        r = row_of[:, j]
        m = r >= 0
        y[m] += g[m, j][:, None] * o_perm[r[m]]
    if y_shared is not None:
        y = y + y_shared
    return y


def combine_backward(dy, o_perm, row_of, g):
    """do[row(t, j)] = g[t, j] dy[t]; dg[t, j] = <dy[t], o[row(t, j)]>, 0 if
    dropped ([EPDP] 三.3: gradients routed back to the experts)."""
    T, k = row_of.shape
    n = o_perm.shape[0]
    do = np.zeros((n, dy.shape[1]), dtype=np.float64)
    dg = np.zeros((T, k), dtype=np.float64)
    for j in range(k):
        r = row_of[:, j]
        m = r >= 0
        do[r[m]] = g[m, j][:, None] * dy[m]
        dg[m, j] = np.sum(dy[m] * o_perm[r[m]], axis=1)
    return do, dg


# --------------------------------------------------------------------------
# router backward  [EPDP 三.4: router (gate) gradients exist and are reduced]
# --------------------------------------------------------------------------
def gating_backward(logits, idx, dg, gating: str) -> np.ndarray:
    """dlogits from dg through the gate-weight Jacobian.

    softmax_topk:  with dp[e] = dg_j where e = e_j, else 0,
                   dl[e] = p[e] * (dp[e] - sum_m p[m] dp[m]),  p = softmax(l)
    renorm / topk_softmax (both are a softmax over the chosen logits):
                   dl[e_j] = g_j * (dg_j - sum_m g_m dg_m), 0 off the chosen set
    The router bias is a constant and gets no gradient.
    """
    T, E = logits.shape
    dl = np.zeros((T, E), dtype=np.float64)
    rows = np.arange(T)[:, None]
    if gating == "softmax_topk":
        p = softmax(logits, axis=1)
        dp = np.zeros((T, E), dtype=np.float64)
        dp[rows, idx] = dg
        dl = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
    elif gating in ("softmax_topk_renorm", "topk_softmax"):
        g = gate_weights(logits, idx, gating)
        s = np.sum(g * dg, axis=1, keepdims=True)
        dl[rows, idx] = g * (dg - s)
    else:
        raise ValueError(gating)
    return dl


def router_backward(x, w_router, dlogits):
    """dW_r = x^T dlogits; router part of dx = dlogits W_r^T."""
    return x.T @ dlogits, dlogits @ w_router.T


# --------------------------------------------------------------------------
# load-balancing loss  [FW: DeepSpeed's moe block takes a "loss_coef", the
# load-balancing loss coefficient; the model config of 实践 四 an
# "aux_loss_factor"; 实践 七.3 负载均衡: the logged auxiliary loss should be
# close to 0 with every expert chosen about equally often]
# --------------------------------------------------------------------------
def balance_loss(logits, idx, E: int, coef: float) -> float:
    """Auxiliary balance loss.  The pages give its coefficient and its goal,
    not its formula; the reading adopted is the usual product of the two
    per-expert loads:

        L = coef * E * sum_e f_e * P_e

    f_e: the share of the T*k routing choices that picked expert e (before
    capacity, so drops do not hide an overloaded expert);
    P_e: the mean over tokens of softmax(l_t)[e], bias included.
    With every expert chosen equally often (f_e = 1/E) L = coef, small for the
    pages' coefficients (0.01 - 0.1); when the choices pile onto the experts
    the router favours, L grows towards coef * E / k."""
    T, k = idx.shape
    f = np.bincount(np.asarray(idx).ravel(), minlength=E).astype(np.float64) / (T * k)
    P = softmax(np.asarray(logits, dtype=np.float64), axis=1).mean(axis=0)
    return float(coef * E * np.sum(f * P))


def balance_loss_grad(logits, idx, E: int, coef: float) -> np.ndarray:
    """dL/dl[t, j] of balance_loss: f is piecewise constant in the logits, so
    only P_e moves, and through the softmax Jacobian
        dL/dl[t, j] = coef * E / T * p[t, j] * (f_j - sum_e f_e p[t, e])."""
    T, k = idx.shape
    f = np.bincount(np.asarray(idx).ravel(), minlength=E).astype(np.float64) / (T * k)
    p = softmax(np.asarray(logits, dtype=np.float64), axis=1)
    return coef * E / T * p * (f[None, :] - (p @ f)[:, None])


def unpermute_sum(dxp, row_of) -> np.ndarray:
    """dx[t] = sum over kept j of dxp[row(t, j)] (sequence order restored,
    [EP] 二 step 4)."""
    T, k = row_of.shape
    dx = np.zeros((T, dxp.shape[1]), dtype=np.float64)
    for j in range(k):
        r = row_of[:, j]
        m = r >= 0
        dx[m] += dxp[r[m]]
    return dx


# --------------------------------------------------------------------------
# whole layer
# --------------------------------------------------------------------------
def _expert_weights(w, e):
    return None if w is None else w[e]


def layer_forward_backward(x, w_router, bias, w1, w_up, w2, dy, *, k: int,
                           gating: str, act: str, capacity_factor: float,
                           ep_ranks: int = 1, placement: str = "contiguous",
                           ws_gate=None, ws_up=None, ws_down=None,
                           n_shared: int = 0, logits=None,
                           backward: bool = True, aux_coef: float = 0.0) -> dict:
    """Forward and backward of the layer on float64 inputs.

    x [T, d], w_router [d, E], bias [E] or None, w1 / w_up [E, d, F],
    w2 [E, F, d], dy [T, d]; shared weights concatenated along the hidden
    axis (ws_gate / ws_up [d, n_shared*Fs], ws_down [n_shared*Fs, d]).
    If ``logits`` is given (e.g. the fp32 logits another implementation
    produced), routing decisions are taken on those values; the layer's own
    gate product is still returned as ``logits_ref``.
    With aux_coef != 0 the balance loss (balance_loss) is returned as
    ``aux_loss`` and the backward differentiates <dy, y> + aux_loss.
    """
    T, d = x.shape
    E = w_router.shape[1]
    out = {}
    out["logits_ref"] = gate_logits(x, w_router, bias)
    lg = out["logits_ref"] if logits is None else np.asarray(logits, dtype=np.float64)
    out["logits"] = lg
    idx = select_topk(lg, k)
    g = gate_weights(lg, idx, gating)
    C = capacity(T, E, k, capacity_factor)
    lay = dispatch_layout(idx, E, C, ep_ranks, placement)
    out.update(topk_idx=idx, topk_w=g, C=C, layout=lay)
    out["aux_loss"] = balance_loss(lg, idx, E, aux_coef) if aux_coef else 0.0
    xp = permute_rows(x, lay, k)
    out["x_perm"] = xp
    n = lay["n"]
    off = lay["expert_offsets"]
    order = lay["slot_expert"]
    o_perm = np.zeros((n, d), dtype=np.float64)
    per_expert = {}
    for s in range(E):
        e = int(order[s])
        r0, r1 = int(off[s]), int(off[s + 1])
        f = expert_ffn_forward(xp[r0:r1], w1[e], w2[e], act, _expert_weights(w_up, e))
        o_perm[r0:r1] = f["o"]
        per_expert[e] = f
    out["o_perm"] = o_perm
    out["per_expert"] = per_expert
    y_shared = None
    shared = []
    if n_shared > 0:
        Fs = ws_gate.shape[1] // n_shared
        y_shared = np.zeros((T, d), dtype=np.float64)
        for s in range(n_shared):
            cols = slice(s * Fs, (s + 1) * Fs)
            f = expert_ffn_forward(x, ws_gate[:, cols], ws_down[cols, :], act,
                                   None if ws_up is None else ws_up[:, cols])
            y_shared += f["o"]
            shared.append(f)
        out["y_shared"] = y_shared
    out["shared"] = shared
    out["y"] = combine(o_perm, lay["row_of"].reshape(T, k), g, y_shared)
    if not backward:
        return out

    row_of = lay["row_of"].reshape(T, k)
    do_perm, dg = combine_backward(dy, o_perm, row_of, g)
    out["do_perm"] = do_perm
    out["d_topk_w"] = dg
    dxp = np.zeros((n, d), dtype=np.float64)
    F = w1.shape[2]
    dw1 = np.zeros_like(w1, dtype=np.float64)
    dw2 = np.zeros_like(w2, dtype=np.float64)
    dwu = None if w_up is None else np.zeros_like(w_up, dtype=np.float64)
    for s in range(E):
        e = int(order[s])
        r0, r1 = int(off[s]), int(off[s + 1])
        b = expert_ffn_backward(xp[r0:r1], do_perm[r0:r1], w1[e], w2[e], act,
                                _expert_weights(w_up, e))
        dxp[r0:r1] = b["dxp"]
        dw1[e] = b["dw_in"]
        dw2[e] = b["dw_out"]
        if dwu is not None:
            dwu[e] = b["dw_up"]
    out.update(dx_perm=dxp, dw1=dw1, dw2=dw2, dw_up=dwu)
    dx_shared = None
    if n_shared > 0:
        Fs = ws_gate.shape[1] // n_shared
        dx_shared = np.zeros((T, d), dtype=np.float64)
        dwsg = np.zeros_like(ws_gate, dtype=np.float64)
        dwsd = np.zeros_like(ws_down, dtype=np.float64)
        dwsu = None if ws_up is None else np.zeros_like(ws_up, dtype=np.float64)
        for s in range(n_shared):
            cols = slice(s * Fs, (s + 1) * Fs)
            b = expert_ffn_backward(x, dy, ws_gate[:, cols], ws_down[cols, :], act,
                                    None if ws_up is None else ws_up[:, cols])
            dx_shared += b["dxp"]
            dwsg[:, cols] = b["dw_in"]
            dwsd[cols, :] = b["dw_out"]
            if dwsu is not None:
                dwsu[:, cols] = b["dw_up"]
        out.update(dx_shared=dx_shared, dws_gate=dwsg, dws_up=dwsu, dws_down=dwsd)
    dl = gating_backward(lg, idx, dg, gating)
    if aux_coef:
        dl = dl + balance_loss_grad(lg, idx, E, aux_coef)
    dwr, dx_router = router_backward(x, w_router, dl)
    out.update(dlogits=dl, dw_router=dwr, dx_router=dx_router)
    dx = unpermute_sum(dxp, row_of) + dx_router
    if dx_shared is not None:
        dx = dx + dx_shared
    out["dx"] = dx
    return out


def layer_from_inputs(inp, logits=None, backward: bool = True) -> dict:
    """Run layer_forward_backward on a synth.LayerInputs (widened to f64)."""
    wl = inp.wl
    return layer_forward_backward(
        to_f64(inp.x), to_f64(inp.w_router),
        None if inp.bias is None else to_f64(inp.bias),
        to_f64(inp.w1), to_f64(inp.w_up), to_f64(inp.w2), to_f64(inp.dy),
        k=wl.k, gating=wl.gating, act=wl.act,
        capacity_factor=wl.capacity_factor, ep_ranks=wl.ep_ranks,
        placement=wl.placement, ws_gate=to_f64(inp.ws_gate),
        ws_up=to_f64(inp.ws_up), ws_down=to_f64(inp.ws_down),
        n_shared=wl.n_shared, logits=logits, backward=backward,
        aux_coef=getattr(wl, "aux_coef", 0.0))
