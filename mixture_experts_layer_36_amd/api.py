"""Thin Python binding of libmoe: one function per C entry point, same names.

Arguments are torch tensors on the GPU (or None for nullable pointers); the
functions only marshal pointers and the current HIP stream into the C call.
No step of the computation runs in Python or PyTorch.
"""
from __future__ import annotations

import ctypes

import torch

from ._native import MoeConfig, MoeGroups, call, plan  # noqa: F401


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libmoe takes device tensors")
    if not t.is_contiguous():
        raise ValueError("libmoe takes contiguous tensors")
    return t.data_ptr()


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def groups(n_groups: int, ffn: int, rows_max: int, offsets: torch.Tensor, use_placement: bool,
           ends: torch.Tensor = None) -> MoeGroups:
    if offsets.dtype != torch.int64 or (ends is not None and ends.dtype != torch.int64):
        raise ValueError("group offsets are int64")
    return MoeGroups(groups=n_groups, ffn=ffn, rows_max=rows_max, offsets=_ptr(offsets),
                     use_placement=1 if use_placement else 0, ends=_ptr(ends))


def moe_route(cfg, x, w_router, bias, logits, topk_idx, topk_w, ws, stream=None):
    call("moe_route", ctypes.byref(cfg), _ptr(x), _ptr(w_router), _ptr(bias), _ptr(logits),
         _ptr(topk_idx), _ptr(topk_w), _ptr(ws), _stream(stream))


def moe_dispatch(cfg, x, topk_idx, x_perm, row_of, assign_of_row, raw_counts, expert_counts,
                 expert_offsets, send_counts, send_offsets, ws, stream=None):
    call("moe_dispatch", ctypes.byref(cfg), _ptr(x), _ptr(topk_idx), _ptr(x_perm), _ptr(row_of),
         _ptr(assign_of_row), _ptr(raw_counts), _ptr(expert_counts), _ptr(expert_offsets),
         _ptr(send_counts), _ptr(send_offsets), _ptr(ws), _stream(stream))


def moe_dispatch_noalloc(cfg, x, topk_idx, x_perm, row_of, assign_of_row, raw_counts, expert_counts,
                         expert_offsets, send_counts, send_offsets, stream=None):
    call("moe_dispatch_noalloc", ctypes.byref(cfg), _ptr(x), _ptr(topk_idx), _ptr(x_perm), _ptr(row_of),
         _ptr(assign_of_row), _ptr(raw_counts), _ptr(expert_counts), _ptr(expert_offsets),
         _ptr(send_counts), _ptr(send_offsets), _stream(stream))


def moe_expert_ffn_fwd(cfg, grp, x_rows, w_in, w_up, w_out, act_saved, h, y_rows, stream=None):
    call("moe_expert_ffn_fwd", ctypes.byref(cfg), ctypes.byref(grp), _ptr(x_rows), _ptr(w_in),
         _ptr(w_up), _ptr(w_out), _ptr(act_saved), _ptr(h), _ptr(y_rows), _stream(stream))


def moe_expert_ffn_bwd(cfg, grp, x_rows, w_in, w_up, w_out, act_saved, h, dy_rows, dx_rows,
                       dw_in, dw_up, dw_out, ws, stream=None):
    call("moe_expert_ffn_bwd", ctypes.byref(cfg), ctypes.byref(grp), _ptr(x_rows), _ptr(w_in),
         _ptr(w_up), _ptr(w_out), _ptr(act_saved), _ptr(h), _ptr(dy_rows), _ptr(dx_rows),
         _ptr(dw_in), _ptr(dw_up), _ptr(dw_out), _ptr(ws), _stream(stream))


def moe_expert_ffn_bwd_data(cfg, grp, w_in, w_up, w_out, act_saved, dy_rows, dx_rows, ws, stream=None):
    call("moe_expert_ffn_bwd_data", ctypes.byref(cfg), ctypes.byref(grp), _ptr(w_in), _ptr(w_up), _ptr(w_out),
         _ptr(act_saved), _ptr(dy_rows), _ptr(dx_rows), _ptr(ws), _stream(stream))


def moe_expert_ffn_bwd_weights(cfg, grp, x_rows, h, dy_rows, dw_in, dw_up, dw_out, ws, stream=None):
    call("moe_expert_ffn_bwd_weights", ctypes.byref(cfg), ctypes.byref(grp), _ptr(x_rows), _ptr(h),
         _ptr(dy_rows), _ptr(dw_in), _ptr(dw_up), _ptr(dw_out), _ptr(ws), _stream(stream))


def moe_expert_ffn_fwd_fused(cfg, grp, x, assign_of_row, topk_w, w_in, w_up, w_out, h, y_tok, stream=None):
    call("moe_expert_ffn_fwd_fused", ctypes.byref(cfg), ctypes.byref(grp), _ptr(x), _ptr(assign_of_row),
         _ptr(topk_w), _ptr(w_in), _ptr(w_up), _ptr(w_out), _ptr(h), _ptr(y_tok), _stream(stream))


def moe_combine_fused(cfg, y_tok, row_of, y_shared, y, stream=None):
    call("moe_combine_fused", ctypes.byref(cfg), _ptr(y_tok), _ptr(row_of), _ptr(y_shared), _ptr(y),
         _stream(stream))


def moe_permute(cfg, x, row_of, x_perm, stream=None):
    call("moe_permute", ctypes.byref(cfg), _ptr(x), _ptr(row_of), _ptr(x_perm), _stream(stream))


def moe_chunk_rows(cfg, topk_idx, row_of, expert_offsets, token_bounds, chunk_rows, stream=None):
    """token_bounds: host sequence of chunks + 1 token indices."""
    n = len(token_bounds) - 1
    bounds = (ctypes.c_int64 * (n + 1))(*[int(b) for b in token_bounds])
    call("moe_chunk_rows", ctypes.byref(cfg), _ptr(topk_idx), _ptr(row_of), _ptr(expert_offsets),
         ctypes.c_int64(n), bounds, _ptr(chunk_rows), _stream(stream))


def moe_combine(cfg, y_perm, row_of, topk_w, y_shared, y, stream=None):
    call("moe_combine", ctypes.byref(cfg), _ptr(y_perm), _ptr(row_of), _ptr(topk_w),
         _ptr(y_shared), _ptr(y), _stream(stream))


def moe_combine_bwd(cfg, dy, y_perm, row_of, topk_w, dy_perm, d_topk_w, stream=None):
    call("moe_combine_bwd", ctypes.byref(cfg), _ptr(dy), _ptr(y_perm), _ptr(row_of),
         _ptr(topk_w), _ptr(dy_perm), _ptr(d_topk_w), _stream(stream))


def moe_route_bwd(cfg, x, logits, topk_idx, d_topk_w, dlogits_add, dlogits, dw_router, ws, stream=None):
    call("moe_route_bwd", ctypes.byref(cfg), _ptr(x), _ptr(logits), _ptr(topk_idx),
         _ptr(d_topk_w), _ptr(dlogits_add), _ptr(dlogits), _ptr(dw_router), _ptr(ws), _stream(stream))


def moe_aux_loss(cfg, logits, raw_counts, coef, loss, ws, stream=None):
    call("moe_aux_loss", ctypes.byref(cfg), _ptr(logits), _ptr(raw_counts), ctypes.c_float(coef),
         _ptr(loss), _ptr(ws), _stream(stream))


def moe_aux_loss_bwd(cfg, logits, raw_counts, coef, dlogits_aux, stream=None):
    call("moe_aux_loss_bwd", ctypes.byref(cfg), _ptr(logits), _ptr(raw_counts), ctypes.c_float(coef),
         _ptr(dlogits_aux), _stream(stream))


def moe_dispatch_bwd(cfg, dx_perm, row_of, dlogits, w_router, dx_add, dx, stream=None):
    call("moe_dispatch_bwd", ctypes.byref(cfg), _ptr(dx_perm), _ptr(row_of), _ptr(dlogits),
         _ptr(w_router), _ptr(dx_add), _ptr(dx), _stream(stream))
