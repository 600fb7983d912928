"""One MoE layer step through libmoe: buffers plus the call sequence.

``MoELayer`` allocates every output and scratch buffer once (torch device
memory, following the "pre-allocate and reuse buffers" advice of the
tutorial's 通信优化方法 section) and issues the C entry points in order:

  forward : moe_route -> moe_dispatch (-> moe_aux_loss) -> moe_expert_ffn_fwd
            (routed, then shared experts) -> moe_combine
  backward: moe_combine_bwd -> moe_expert_ffn_bwd (routed, then shared)
            (-> moe_aux_loss_bwd) -> moe_route_bwd -> moe_dispatch_bwd

With aux_coef != 0 the step also computes the balance loss (DeepSpeed's
loss_coef in the tutorial's framework section) and differentiates it with
upstream gradient 1, alongside <dy, y>.

All of it is enqueued on one stream with no host synchronisation.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import torch

from . import api
from ._native import make_config, plan

TORCH_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


@dataclass
class Weights:
    w_router: torch.Tensor                 # [d, E]
    w1: torch.Tensor                       # [E, d, F]  (W1 or W_gate)
    w2: torch.Tensor                       # [E, F, d]  (W2 or W_down)
    w_up: Optional[torch.Tensor] = None    # [E, d, F]  (SwiGLU)
    bias: Optional[torch.Tensor] = None    # [E] fp32
    ws_gate: Optional[torch.Tensor] = None  # [d, n_shared*Fs]
    ws_up: Optional[torch.Tensor] = None
    ws_down: Optional[torch.Tensor] = None  # [n_shared*Fs, d]


class MoELayer:
    def __init__(self, T, d, ffn, E, k, capacity_factor, gating, act, dtype, ep_ranks=1,
                 placement="contiguous", n_shared=0, ffn_shared=0, device="cuda", aux_coef=0.0):
        self.cfg = make_config(T, d, ffn, E, k, capacity_factor, gating, act, dtype, ep_ranks,
                               placement, n_shared, ffn_shared)
        self.sizes = plan(self.cfg)
        self.T, self.d, self.F, self.E, self.k = T, d, ffn, E, k
        self.R = ep_ranks
        self.act = act
        self.n_shared = n_shared
        self.Fs = n_shared * ffn_shared
        dt = TORCH_DTYPES[dtype]
        self.dtype = dt
        dev = torch.device(device)
        self.device = dev
        n = self.sizes.n_max
        m = 2 if act == "swiglu" else 1
        e = lambda *s, dtype=dt: torch.empty(*s, dtype=dtype, device=dev)  # noqa: E731
        # forward outputs
        self.logits = e(T, E, dtype=torch.float32)
        self.topk_idx = e(T, k, dtype=torch.int32)
        self.topk_w = e(T, k, dtype=torch.float32)
        self.x_perm = e(max(n, 1), d)
        self.row_of = e(T * k, dtype=torch.int32)
        self.assign_of_row = e(max(n, 1), dtype=torch.int32)
        self.raw_counts = e(E, dtype=torch.int32)
        self.expert_counts = e(E, dtype=torch.int32)
        self.expert_offsets = e(E + 1, dtype=torch.int64)
        self.send_counts = e(ep_ranks, dtype=torch.int32)
        self.send_offsets = e(ep_ranks + 1, dtype=torch.int64)
        self.act_saved = e(max(n, 1), m * ffn)
        self.h = e(max(n, 1), ffn)
        self.y_perm = e(max(n, 1), d)
        self.y = e(T, d)
        # backward outputs
        self.dy_perm = e(max(n, 1), d)
        self.d_topk_w = e(T, k, dtype=torch.float32)
        self.dx_perm = e(max(n, 1), d)
        self.dw1 = e(E, d, ffn)
        self.dw_up = e(E, d, ffn) if act == "swiglu" else None
        self.dw2 = e(E, ffn, d)
        self.dlogits = e(T, E, dtype=torch.float32)
        self.dw_router = e(d, E)
        self.dx = e(T, d)
        if n_shared > 0:
            self.s_offsets = torch.tensor([0, T], dtype=torch.int64, device=dev)
            self.s_act = e(T, m * self.Fs)
            self.s_h = e(T, self.Fs)
            self.y_shared = e(T, d)
            self.dx_shared = e(T, d)
            self.dws_gate = e(d, self.Fs)
            self.dws_up = e(d, self.Fs) if act == "swiglu" else None
            self.dws_down = e(self.Fs, d)
        self.aux_coef = float(aux_coef)
        if self.aux_coef:
            self.aux_loss = e(1, dtype=torch.float32)
            self.dlogits_aux = e(T, E, dtype=torch.float32)
        self.ws = e(max(1, (self.sizes.workspace_bytes + 255) // 256 * 256), dtype=torch.uint8)
        self.grp = api.groups(E, ffn, n, self.expert_offsets, use_placement=True)
        if n_shared > 0:
            self.sgrp = api.groups(1, self.Fs, T, self.s_offsets, use_placement=False)

    # ------------------------------------------------------------------ steps
    def route(self, x, w: Weights):
        api.moe_route(self.cfg, x, w.w_router, w.bias, self.logits, self.topk_idx, self.topk_w, self.ws)

    def dispatch(self, x):
        api.moe_dispatch(self.cfg, x, self.topk_idx, self.x_perm, self.row_of, self.assign_of_row,
                         self.raw_counts, self.expert_counts, self.expert_offsets, self.send_counts,
                         self.send_offsets, self.ws)

    def experts_fwd(self, w: Weights):
        api.moe_expert_ffn_fwd(self.cfg, self.grp, self.x_perm, w.w1, w.w_up, w.w2, self.act_saved,
                               self.h, self.y_perm)

    def shared_fwd(self, x, w: Weights):
        api.moe_expert_ffn_fwd(self.cfg, self.sgrp, x, w.ws_gate, w.ws_up, w.ws_down, self.s_act,
                               self.s_h, self.y_shared)

    def combine(self):
        api.moe_combine(self.cfg, self.y_perm, self.row_of, self.topk_w,
                        self.y_shared if self.n_shared else None, self.y)

    def combine_bwd(self, dy):
        api.moe_combine_bwd(self.cfg, dy, self.y_perm, self.row_of, self.topk_w, self.dy_perm,
                            self.d_topk_w)

    def experts_bwd(self, w: Weights):
        api.moe_expert_ffn_bwd(self.cfg, self.grp, self.x_perm, w.w1, w.w_up, w.w2, self.act_saved,
                               self.h, self.dy_perm, self.dx_perm, self.dw1, self.dw_up, self.dw2,
                               self.ws)

    def shared_bwd(self, x, dy, w: Weights):
        api.moe_expert_ffn_bwd(self.cfg, self.sgrp, x, w.ws_gate, w.ws_up, w.ws_down, self.s_act,
                               self.s_h, dy, self.dx_shared, self.dws_gate, self.dws_up,
                               self.dws_down, self.ws)

    def aux_fwd(self):
        api.moe_aux_loss(self.cfg, self.logits, self.raw_counts, self.aux_coef, self.aux_loss, self.ws)

    def aux_bwd(self):
        api.moe_aux_loss_bwd(self.cfg, self.logits, self.raw_counts, self.aux_coef, self.dlogits_aux)

    def route_bwd(self, x):
        api.moe_route_bwd(self.cfg, x, self.logits, self.topk_idx, self.d_topk_w,
                          self.dlogits_aux if self.aux_coef else None, self.dlogits, self.dw_router, self.ws)

    def dispatch_bwd(self, w: Weights):
        api.moe_dispatch_bwd(self.cfg, self.dx_perm, self.row_of, self.dlogits, w.w_router,
                             self.dx_shared if self.n_shared else None, self.dx)

    def forward(self, x, w: Weights):
        self.route(x, w)
        self.dispatch(x)
        if self.aux_coef:
            self.aux_fwd()
        self.experts_fwd(w)
        if self.n_shared:
            self.shared_fwd(x, w)
        self.combine()
        return self.y

    def backward(self, x, dy, w: Weights):
        self.combine_bwd(dy)
        self.experts_bwd(w)
        if self.n_shared:
            self.shared_bwd(x, dy, w)
        if self.aux_coef:
            self.aux_bwd()
        self.route_bwd(x)
        self.dispatch_bwd(w)
        return self.dx

    def step(self, x, dy, w: Weights):
        self.forward(x, w)
        self.backward(x, dy, w)

    # ---------------------------------------------------------- fused forward
    def forward_fused(self, x, w: Weights):
        """Forward-only pass through the fused path (Tutel's fused kernels in
        the tutorial's framework section): the layout without the dispatch
        copy, GEMM-1 gathering its rows from x through assign_of_row and
        keeping only h, GEMM-2 writing weighted, un-permuted rows, and a
        plain k-row sum.  y equals forward()'s within rounding (each row is
        weighted before its bf16 rounding instead of after)."""
        if getattr(self, "y_tok", None) is None:
            self.y_tok = torch.empty(self.T * self.k, self.d, dtype=self.dtype, device=self.device)
        self.route(x, w)
        api.moe_dispatch(self.cfg, None, self.topk_idx, None, self.row_of, self.assign_of_row, self.raw_counts,
                         self.expert_counts, self.expert_offsets, self.send_counts, self.send_offsets, self.ws)
        api.moe_expert_ffn_fwd_fused(self.cfg, self.grp, x, self.assign_of_row, self.topk_w, w.w1, w.w_up, w.w2,
                                     self.h, self.y_tok)
        if self.n_shared:
            self.shared_fwd(x, w)
        api.moe_combine_fused(self.cfg, self.y_tok, self.row_of, self.y_shared if self.n_shared else None, self.y)
        return self.y

    # ------------------------------------------------------------ pipelined
    def _pipeline_setup(self, chunks):
        """Per-chunk configs (the same layer over a token range, for the
        token-range calls; the expert FFN calls keep the layer's config, as
        their group tables address the whole row buffers) and buffers:
        the chunk row table, a second workspace for the side stream's router
        backward, the side stream and its events."""
        if getattr(self, "_pipe_chunks", None) == chunks:
            return
        T, E = self.T, self.E
        self._bounds = [T * r // chunks for r in range(chunks + 1)]
        self._ccfg = [make_config(self._bounds[r + 1] - self._bounds[r], self.d, self.F, E, self.k,
                                  self.cfg.capacity_factor, self.cfg.gating, self.cfg.act, self.cfg.dtype,
                                  self.R, self.cfg.placement, self.cfg.n_shared, self.cfg.ffn_shared)
                      for r in range(chunks)]
        self.chunk_rows = torch.empty((chunks + 1) * E, dtype=torch.int64, device=self.device)
        n = self.sizes.n_max
        self._cgrp = [api.groups(E, self.F, n, self.chunk_rows[r * E:(r + 1) * E], True,
                                 ends=self.chunk_rows[(r + 1) * E:(r + 2) * E]) for r in range(chunks)]
        self.ws2 = torch.empty_like(self.ws)
        self._side = torch.cuda.Stream(device=self.device)
        self._pipe_chunks = chunks

    def step_pipelined(self, x, dy, w: Weights, chunks=2):
        """One step with the batch cut into `chunks` token chunks on two
        streams (FlowMoE notes, 关键设计: pipelining over token chunks;
        tutorial, 通信优化方法 三: overlap communication with computation).
        The bandwidth kernels of a chunk (permute, combine, combine backward,
        dispatch backward) run on a side stream beside the expert GEMMs of
        the other chunks on the main stream.

        Routing and the dispatch layout cover the whole batch first (every
        expert's segment start needs every token's choice); since each
        expert's kept rows are in token order, chunk r owns a contiguous
        sub-range of every segment (moe_chunk_rows), so the chunks' GEMMs
        run on sub-range group tables over the same buffers, and the weight
        gradients once over whole groups.  Every output is bit-identical to
        step().  The backward starts after the forward has finished, as it
        would when dy arrives from the next layer."""
        chunks = max(1, min(int(chunks), self.T, 16))
        self._pipeline_setup(chunks)
        main, side = torch.cuda.current_stream(), self._side
        k, b = self.k, self._bounds
        ev = lambda: torch.cuda.Event()  # noqa: E731

        def rec(stream):
            e = ev()
            e.record(stream)
            return e

        # forward: whole-batch routing and layout, then the chunks
        self.route(x, w)
        api.moe_dispatch(self.cfg, None, self.topk_idx, None, self.row_of, self.assign_of_row, self.raw_counts,
                         self.expert_counts, self.expert_offsets, self.send_counts, self.send_offsets, self.ws, main)
        if self.aux_coef:
            self.aux_fwd()
        api.moe_chunk_rows(self.cfg, self.topk_idx, self.row_of, self.expert_offsets, b, self.chunk_rows, main)
        side.wait_event(rec(main))
        perm = []
        for r in range(chunks):
            api.moe_permute(self._ccfg[r], x[b[r]:b[r + 1]], self.row_of[b[r] * k:b[r + 1] * k], self.x_perm, side)
            perm.append(rec(side))
        if self.n_shared:
            self.shared_fwd(x, w)
        ffn = []
        for r in range(chunks):
            main.wait_event(perm[r])
            api.moe_expert_ffn_fwd(self.cfg, self._cgrp[r], self.x_perm, w.w1, w.w_up, w.w2, self.act_saved,
                                   self.h, self.y_perm, main)
            ffn.append(rec(main))
        for r in range(chunks):
            side.wait_event(ffn[r])
            api.moe_combine(self._ccfg[r], self.y_perm, self.row_of[b[r] * k:b[r + 1] * k],
                            self.topk_w[b[r]:b[r + 1]], self.y_shared[b[r]:b[r + 1]] if self.n_shared else None,
                            self.y[b[r]:b[r + 1]], side)
        # the forward is complete before the backward starts
        main.wait_event(rec(side))
        side.wait_event(rec(main))
        cb = []
        for r in range(chunks):
            api.moe_combine_bwd(self._ccfg[r], dy[b[r]:b[r + 1]], self.y_perm, self.row_of[b[r] * k:b[r + 1] * k],
                                self.topk_w[b[r]:b[r + 1]], self.dy_perm, self.d_topk_w[b[r]:b[r + 1]], side)
            cb.append(rec(side))
        if self.aux_coef:
            api.moe_aux_loss_bwd(self.cfg, self.logits, self.raw_counts, self.aux_coef, self.dlogits_aux, side)
        api.moe_route_bwd(self.cfg, x, self.logits, self.topk_idx, self.d_topk_w,
                          self.dlogits_aux if self.aux_coef else None, self.dlogits, self.dw_router, self.ws2, side)
        if self.n_shared:
            self.shared_bwd(x, dy, w)
        dg = []
        for r in range(chunks):
            main.wait_event(cb[r])
            api.moe_expert_ffn_bwd_data(self.cfg, self._cgrp[r], w.w1, w.w_up, w.w2, self.act_saved,
                                        self.dy_perm, self.dx_perm, self.ws, main)
            dg.append(rec(main))
        api.moe_expert_ffn_bwd_weights(self.cfg, self.grp, self.x_perm, self.h, self.dy_perm, self.dw1, self.dw_up,
                                       self.dw2, self.ws, main)
        for r in range(chunks):
            side.wait_event(dg[r])
            api.moe_dispatch_bwd(self._ccfg[r], self.dx_perm, self.row_of[b[r] * k:b[r + 1] * k],
                                 self.dlogits[b[r]:b[r + 1]], w.w_router,
                                 self.dx_shared[b[r]:b[r + 1]] if self.n_shared else None, self.dx[b[r]:b[r + 1]],
                                 side)
        main.wait_event(rec(side))

    def capture_step(self, x, dy, w: Weights):
        """Record one whole step (every entry point, forward and backward) into
        a HIP graph; replaying it re-runs the step on the same buffers, with
        one launch from the host instead of one per kernel.  The entry points
        launch only the library's own kernels (no memory sets, allocations or
        synchronisation), so the step captures whole.  A first step runs on a
        side stream before the capture, so that every launcher's one-time
        set-up (kernel attributes) happens outside it."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self.step(x, dy, w)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            self.step(x, dy, w)
        torch.cuda.synchronize()
        return graph
