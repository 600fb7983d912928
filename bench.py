#!/usr/bin/env python3
"""Benchmark of one MoE layer step (forward + backward) on one MI355X.

A step runs every stage of the path on one batch of synthetic input already
resident in HBM: route, dispatch (with the EP send layout), grouped expert
FFN forward (routed, then shared experts), combine, combine backward, grouped
expert FFN backward, router backward, dispatch backward.

Prints ONE JSON line (stdout):
  value       tokens per second of the whole step (T / step time)
  roofline    the grouped expert GEMM (all its launches in a step): algorithmic
              FLOPs (3 x 2 n d F m, plus shared experts) / its event-measured
              time, against the bf16 dense MFMA peak; `traffic` is the HBM
              bytes per step of those launches from hardware counters
              (profiles/gemm_traffic_<workload>.txt), reported only while the
              GEMM sources still hash to the ones the counters were taken on
  cpu_baseline the CPU oracle timed on a bounded sample of the same workload
  kernels     per-entry-point times and achieved rates (events around each call)

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload mixtral_bf16]
       [--graph]                (time replays of the step captured in one HIP graph)
       [--calibrate-copy MIB]   (also runs a plain device copy of MIB MiB, for
                                 scaling memory counters in a profiler run)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

PEAK_HBM_GBS = 8000.0
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


GEMM_SOURCES = ("gemm3.hip", "gemm_common.h", "gemm_addr.h", "gemm.h", "common.h", "moe_api.hip")


def gemm_source_hash():
    """sha256 over the sources that define the grouped GEMM kernels and their launches."""
    h = hashlib.sha256()
    for name in GEMM_SOURCES:
        with open(os.path.join(HERE, "mixture_experts_layer_36_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def gemm_traffic(workload):
    """HBM bytes per step of the grouped GEMM launches, from the counter
    summary of this workload, or None when it is missing or was taken on
    other GEMM sources."""
    path = os.path.join(HERE, "profiles", f"gemm_traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.lstrip().startswith("#"):
                key, val = line.split("=", 1)
                kv[key.strip()] = val.strip()
    if kv.get("gemm_source_sha256") != gemm_source_hash():
        return None
    return {"read_bytes": int(kv["read_bytes_per_step"]), "write_bytes": int(kv["write_bytes_per_step"]),
            "bytes": int(kv["read_bytes_per_step"]) + int(kv["write_bytes_per_step"]),
            "source": os.path.relpath(path, HERE)}


def algorithmic(wl, n, T_kept):
    """Algorithmic bytes / FLOPs of each entry point for one step."""
    s = 2 if wl.dtype == "bf16" else 4
    T, d, F, E, k = wl.T, wl.d, wl.ffn, wl.E, wl.k
    m = 3 if wl.act == "swiglu" else 2
    Fs = wl.n_shared * wl.ffn_shared
    out = {}
    out["route"] = dict(bytes=T * d * s + d * E * s + T * E * 4 + 8 * T * k)
    out["dispatch"] = dict(bytes=T_kept * d * s + n * d * s + 8 * T * k + 4 * n)
    out["ffn_fwd"] = dict(flops=2 * n * d * F * m)
    out["combine"] = dict(bytes=n * d * s + T * d * s + (T * d * s if Fs else 0) + 8 * T * k)
    out["combine_bwd"] = dict(bytes=T * d * s + 2 * n * d * s + 12 * T * k)
    out["ffn_bwd"] = dict(flops=2 * 2 * n * d * F * m)
    out["route_bwd"] = dict(bytes=T * d * s + T * E * 4 * 2 + d * E * s + T * k * 8)
    out["dispatch_bwd"] = dict(bytes=n * d * s + T * d * s + (T * d * s if Fs else 0) + T * E * 4 + 4 * T * k
                               + d * E * s)
    if Fs:
        out["shared_fwd"] = dict(flops=2 * T * d * Fs * m)
        out["shared_bwd"] = dict(flops=2 * 2 * T * d * Fs * m)
    return out


def cpu_baseline(wl, inp, n_tokens):
    """Time the oracle (float64 numpy) on the first n_tokens tokens of the
    workload with its full weights, with all host cores available to BLAS."""
    import oracle
    from threadpoolctl import threadpool_info, threadpool_limits
    cores = len(os.sched_getaffinity(0))
    t_s = min(n_tokens, wl.T)
    f = oracle.to_f64
    X, DY = f(inp.x[:t_s]), f(inp.dy[:t_s])
    wr, b = f(inp.w_router), (None if inp.bias is None else f(inp.bias))
    w1, wu, w2 = f(inp.w1), f(inp.w_up), f(inp.w2)
    sg, su, sd = f(inp.ws_gate), f(inp.ws_up), f(inp.ws_down)
    with threadpool_limits(limits=cores):
        info = threadpool_info()
        threads = max([int(i.get("num_threads", 1)) for i in info] or [1])
        t0 = time.perf_counter()
        oracle.layer_forward_backward(X, wr, b, w1, wu, w2, DY, k=wl.k, gating=wl.gating, act=wl.act,
                                      capacity_factor=wl.capacity_factor, ep_ranks=wl.ep_ranks,
                                      placement=wl.placement, ws_gate=sg, ws_up=su, ws_down=sd,
                                      n_shared=wl.n_shared)
        dt = time.perf_counter() - t0
    return {"value": round(t_s / dt, 2), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"float64 oracle fwd+bwd on the first {t_s} of {wl.T} tokens of {wl.name} with the "
                      f"full weights ({dt:.2f} s, {cores} host cores visible)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mixtral_bf16")
    ap.add_argument("--cpu-tokens", type=int, default=2048)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of the whole step captured in one HIP graph instead of eager calls")
    ap.add_argument("--pipeline", type=int, default=0, metavar="CHUNKS",
                    help="time the step with the batch cut into CHUNKS token chunks on two streams")
    ap.add_argument("--fused", action="store_true",
                    help="also time the forward pass alone, unfused and fused (gather prologue, weighted epilogue)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark measures one GPU's share of the layer; "
                                   "it runs on exactly one GPU (--gpus 1)"}))
        return 2

    import torch
    import synth
    from mixture_experts_layer_36_amd import _native
    from mixture_experts_layer_36_amd.layer import MoELayer, Weights

    if not torch.cuda.is_available():
        log("no GPU visible")
        return 1
    _native.load()
    wl = synth.workload(args.workload)
    log(f"[bench] workload {wl.name}: generating inputs")
    inp = synth.make_inputs(wl)

    def dev(a):
        if a is None:
            return None
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(a).cuda()

    layer = MoELayer(wl.T, wl.d, wl.ffn, wl.E, wl.k, wl.capacity_factor, wl.gating, wl.act, wl.dtype,
                     wl.ep_ranks, wl.placement, wl.n_shared, wl.ffn_shared)
    w = Weights(w_router=dev(inp.w_router), w1=dev(inp.w1), w2=dev(inp.w2), w_up=dev(inp.w_up),
                bias=dev(inp.bias), ws_gate=dev(inp.ws_gate), ws_up=dev(inp.ws_up), ws_down=dev(inp.ws_down))
    x, dy = dev(inp.x), dev(inp.dy)
    torch.cuda.synchronize()
    run_step = lambda: layer.step(x, dy, w)  # noqa: E731
    if args.pipeline:
        run_step = lambda: layer.step_pipelined(x, dy, w, chunks=args.pipeline)  # noqa: E731
    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        run_step()
    torch.cuda.synchronize()

    # 1) whole steps, events only at the ends
    if args.graph:
        graph = layer.capture_step(x, dy, w)
        run_step = graph.replay
        for _ in range(args.warmup):
            run_step()
    log(f"[bench] timing {args.steps} steps" + (" (HIP graph replays)" if args.graph else ""))
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(st)
    for _ in range(args.steps):
        run_step()
    e1.record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = e0.elapsed_time(e1) / args.steps

    # 2) per entry point, events around each call (same stream)
    stages = [("route", lambda: layer.route(x, w)), ("dispatch", lambda: layer.dispatch(x)),
              ("ffn_fwd", lambda: layer.experts_fwd(w))]
    if wl.n_shared:
        stages.append(("shared_fwd", lambda: layer.shared_fwd(x, w)))
    stages += [("combine", layer.combine), ("combine_bwd", lambda: layer.combine_bwd(dy)),
               ("ffn_bwd", lambda: layer.experts_bwd(w))]
    if wl.n_shared:
        stages.append(("shared_bwd", lambda: layer.shared_bwd(x, dy, w)))
    stages += [("route_bwd", lambda: layer.route_bwd(x)), ("dispatch_bwd", lambda: layer.dispatch_bwd(w))]
    if args.pipeline:
        # the two halves of the dispatch the pipelined step calls apart
        from mixture_experts_layer_36_amd import api
        stages += [("dispatch_layout", lambda: api.moe_dispatch(
                        layer.cfg, None, layer.topk_idx, None, layer.row_of, layer.assign_of_row, layer.raw_counts,
                        layer.expert_counts, layer.expert_offsets, layer.send_counts, layer.send_offsets, layer.ws)),
                   ("permute", lambda: api.moe_permute(layer.cfg, x, layer.row_of, layer.x_perm))]
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in stages]
           for _ in range(args.steps)]
    for s in range(args.steps):
        for (name, fn), (a, b) in zip(stages, evs[s]):
            a.record(st)
            fn()
            b.record(st)
    torch.cuda.synchronize()
    times = {name: float(np.mean([evs[s][i][0].elapsed_time(evs[s][i][1]) for s in range(args.steps)]))
             for i, (name, _) in enumerate(stages)}

    n = int(layer.expert_offsets[-1].item())
    row_of = layer.row_of.view(wl.T, wl.k)
    T_kept = int((row_of >= 0).any(dim=1).sum().item())
    alg = algorithmic(wl, n, T_kept)
    kernels = {}
    for name, ms in times.items():
        if name not in alg:
            kernels[name] = {"ms": round(ms, 4)}
            continue
        a = alg[name]
        ent = {"ms": round(ms, 4)}
        if "bytes" in a:
            gbs = a["bytes"] / (ms * 1e-3) / 1e9
            ent.update(bytes=a["bytes"], GBps=round(gbs, 1), frac_hbm=round(gbs / PEAK_HBM_GBS, 4))
        else:
            tf = a["flops"] / (ms * 1e-3) / 1e12
            ent.update(flops=a["flops"], TFLOPs=round(tf, 1), frac_mfma=round(tf / PEAK_TFLOPS[wl.dtype], 4))
        kernels[name] = ent
    gemm_names = [k_ for k_ in ("ffn_fwd", "ffn_bwd", "shared_fwd", "shared_bwd") if k_ in times]
    gemm_ms = sum(times[k_] for k_ in gemm_names)
    gemm_flops = sum(alg[k_]["flops"] for k_ in gemm_names)
    launches = 6 * (2 if wl.n_shared else 1)
    achieved = gemm_flops / (gemm_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[wl.dtype]
    # timed as the expert FFN entry points: the split-reduction and weight-transpose
    # kernels inside them count as GEMM time
    roofline = {"kernel": f"grouped expert GEMM, fwd+bwd ({launches} launches per step, with their "
                          "split reductions and weight transposes)",
                "bound": "mfma", "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": None,
                "per_step_flops": gemm_flops, "per_step_ms": round(gemm_ms, 4)}
    traffic = gemm_traffic(wl.name)
    if traffic is not None:
        roofline["traffic"] = traffic["bytes"]
        roofline["traffic_detail"] = traffic
    permute_gbs = kernels["dispatch"]["GBps"]

    if args.calibrate_copy > 0:
        # a plain elementwise copy (read N bytes, write N bytes) of known size
        nbytes = args.calibrate_copy << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy: 3 x neg over {nbytes} bytes (read {nbytes}, write {nbytes} each)")
        del src, dst

    cpu = None
    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline on {args.cpu_tokens} tokens")
        cpu = cpu_baseline(wl, inp, args.cpu_tokens)

    fused = None
    if args.fused:
        # forward only: forward() (dispatch copy, saved activations, weighted
        # combine) against forward_fused() (gather prologue, h only, weighted
        # un-permuted rows, k-row sum); alternating blocks of steps
        fwd = {"unfused": lambda: layer.forward(x, w), "fused": lambda: layer.forward_fused(x, w)}
        samples = {k_: [] for k_ in fwd}
        for fn in fwd.values():
            fn()
        for _ in range(3):
            for key, fn in fwd.items():
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(st)
                for _ in range(args.steps):
                    fn()
                b.record(st)
                torch.cuda.synchronize()
                samples[key].append(a.elapsed_time(b) / args.steps)
        fused = {k_ + "_ms": round(float(np.median(v)), 4) for k_, v in samples.items()}
        fused["tokens_per_s_fused"] = round(wl.T / (fused["fused_ms"] * 1e-3), 1)

    pipeline = None
    if args.pipeline:
        # the pages' overlap model (tutorial, 通信优化方法 三): total = T_A +
        # max(T_comm, T_B), with T_comm the bandwidth kernels the side stream
        # takes, T_B the expert GEMMs, T_A the rest (routing and layout)
        t_comm = sum(times[n_] for n_ in ("permute", "combine", "combine_bwd", "route_bwd", "dispatch_bwd"))
        t_b = gemm_ms
        t_a = times["route"] + times["dispatch_layout"]
        pipeline = {"chunks": args.pipeline, "T_A_ms": round(t_a, 4), "T_comm_ms": round(t_comm, 4),
                    "T_B_ms": round(t_b, 4), "model_ms": round(t_a + max(t_comm, t_b), 4),
                    "serial_ms": round(t_a + t_comm + t_b, 4), "measured_ms": round(ms_step, 4)}

    result = {
        "metric": "MoE layer fwd+bwd tokens/s on 1 MI355X; grouped-GEMM % MFMA peak; permute GB/s",
        "value": round(wl.T / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": wl.name, "T": wl.T, "d": wl.d, "ffn": wl.ffn, "E": wl.E, "k": wl.k,
                   "capacity_factor": wl.capacity_factor, "gating": wl.gating, "act": wl.act,
                   "n_shared": wl.n_shared, "ffn_shared": wl.ffn_shared, "ep_ranks": wl.ep_ranks,
                   "rows_kept": n, "parallelism": "single GPU",
                   "launch": "hip graph" if args.graph else (
                       f"eager, {args.pipeline} token chunks on two streams" if args.pipeline else "eager")},
        "grouped_gemm_frac_mfma": roofline["frac"],
        "permute_GBps": permute_gbs,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "pipeline": pipeline,
        "fused_forward": fused,
        "wall_s_timed": round(wall, 3),
    }
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
