#!/usr/bin/env python3
"""Attention forward benchmark on one MI355X.

    python bench.py [--workload long|bandwidth|compute|launch|tiny|qkv_launch|qkv_bandwidth|...]
                    [--pass fwd|bwd] [--steps K] [--warmup W] [--gpus 1] [--graph G]

One step is one exact attention forward (one launch of the library's kernel)
over a batch of seeded synthetic inputs already resident in device memory.
With no --workload the line is quoted on the long-sequence shape (B=32,
H=16, S=100000, d_h=64, fp16, causal: the largest single-GPU configuration)
and carries sub-records for the bandwidth-, compute- and launch-bound shapes,
each timed on its own kernel with its own roofline and CPU baseline.
Exactly K steps are timed. For the launch-bound shapes the K calls are
submitted as replays of HIP graphs of captured calls (at most G = 100 per
graph, plus one graph for the remainder), so the host's per-call submission
cost is paid once per graph; the eager per-step rate is reported beside it.
Prints ONE JSON line: throughput in TFLOP/s counted on the visible (query,
key) pairs only (4 * d_h flops per pair: two matrix products), the roofline
of the kernel (achieved vs MI355X peak, from HIP events on the stream the
kernel runs on), and the float64 CPU oracle timed on a bounded sample of the
same workload on this host's cores.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0            # MI355X HBM3E, GB/s
PEAK_MFMA_TFLOPS = {"f16": 2516.6, "bf16": 2516.6, "f32": 157.3}  # dense matrix-core peaks
MALL_BYTES = 256 << 20           # working sets below this are rotated over buffer sets

HEADLINE = "long"                # the workload the default line is quoted on
SUBRECORDS = ("bandwidth", "compute", "launch")  # further forward regimes in the same line
SUB_CPU_BUDGET_S = 10.0          # oracle seconds per sub-record
DEFAULT_STEPS = {"tiny": 2000, "launch": 2000, "bandwidth": 100, "compute": 200, "long": 10,
                 "bwd": 50, "bwd_gqa": 50, "qkv_launch": 2000, "qkv_bandwidth": 100, "qkv_heads8": 100}
DEFAULT_WARMUP = {"tiny": 50, "launch": 50, "bandwidth": 5, "compute": 10, "long": 2, "bwd": 5,
                  "bwd_gqa": 5, "qkv_launch": 50, "qkv_bandwidth": 5, "qkv_heads8": 5}
WARMUP_S = 0.5                   # minimum warm-up time before any timed region
DEFAULT_GRAPH = {"tiny": 100, "launch": 100, "bandwidth": 0, "compute": 0, "long": 0, "bwd": 0,
                 "bwd_gqa": 0, "qkv_launch": 100, "qkv_bandwidth": 0, "qkv_heads8": 0}
BOUND = {"tiny": "hbm", "launch": "hbm", "bandwidth": "hbm", "compute": "mfma", "long": "mfma",
         "bwd": "mfma", "bwd_gqa": "mfma"}
# the sources each timed path's kernels are built from (their hash marks
# stored counter runs as current or stale)
KERNEL_SOURCES = ("attn_common.h", "attn_mfma.hip", "attn_short.hip", "attn_short16.hip",
                  "attn_f32.hip", "attn_valu.hip", "launch.h", "mha_api.hip")
QKV_SOURCES = ("attn_common.h", "attn_qkv16.hip", "launch.h", "mha_api.hip")
BWD_SOURCES = ("attn_common.h", "attn_bwd.hip", "launch.h", "mha_api.hip")


def dtype_tag(dt) -> str:
    return {"torch.float16": "f16", "torch.bfloat16": "bf16", "torch.float32": "f32"}[str(dt)]


def pair_count(w, kl_cpu) -> int:
    """Visible (query, key) pairs over all heads, from the drawn key lengths."""
    S = w.S
    Ls = [S] * w.B if kl_cpu is None else [max(0, min(S, int(x))) for x in kl_cpu.tolist()]
    tot = 0
    for L in Ls:
        tot += (L * (L + 1) // 2 + (S - L) * L) if w.causal else S * L
    return tot * w.H


def algorithmic_bytes(w, kl_cpu, esize: int) -> int:
    S, D = w.S, w.D
    Ls = [S] * w.B if kl_cpu is None else [max(0, min(S, int(x))) for x in kl_cpu.tolist()]
    qo = 2 * w.B * w.H * S * D * esize
    kv = 2 * w.H * D * esize * sum(Ls)
    lse = 4 * w.B * w.H * S
    kl = 0 if kl_cpu is None else 4 * w.B
    return qo + kv + lse + kl


def kernel_source_hash(files=KERNEL_SOURCES) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "exact_attention_mha_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def stored_traffic(workload: str, per_launch_src_hash: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != per_launch_src_hash:
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(w, q, k, v, kl, flops_per_pair_unit: int, budget_s: float = 12.0):
    """Time the float64 oracle as it stands on a bounded sample of this workload."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        blas = 1
    avail = len(os.sched_getaffinity(0))
    threads = max(1, min(16, avail))
    # the long workload stays on the device: the oracle copies back only the
    # heads its sampled rows need
    qc, kc, vc = (q, k, v) if w.name == "long" else (q.cpu(), k.cpu(), v.cpu())
    klc = None if kl is None else kl.cpu()
    D = w.D
    if w.name == "long":
        # exact rows of a seeded sample; the sample grows until it takes
        # about half the budget or more (first pass: 256 rows, to size it)
        from workloads import sample_rows
        n = 256
        while True:
            rows = sample_rows(w.B, w.H, w.S, n, seed=0, tile=128, n_heads=4)
            pairs = int(sum(min(int(i) + 1, w.S) for i in rows[:, 2]))
            t0 = time.perf_counter()
            oracle.attention_rows(qc, kc, vc, rows, causal=True, key_len=klc)
            dt = time.perf_counter() - t0
            if dt >= 0.5 * budget_s or n >= 32768:
                break
            n = min(32768, max(2 * n, int(n * budget_s / max(dt, 1e-3))))
        sample = f"{rows.shape[0]} query rows of S={w.S} in 4 heads (exact rows)"
        reps = 1
    else:
        ws = w
        sample = "whole workload, repeated"
        pairs = pair_count(ws, klc)
        reps = 0
        t0 = time.perf_counter()
        while True:
            oracle.attention(qc, kc, vc, causal=w.causal, key_len=klc, threads=threads)
            reps += 1
            dt = time.perf_counter() - t0
            if dt > budget_s:
                break
        sample += f" x{reps}"
    tflops = flops_per_pair_unit * pairs * reps / dt / 1e12
    return {"value": tflops, "unit": "TFLOP/s", "cores": max(blas, threads if w.name != "long" else blas),
            "kind": "oracle", "sample": sample, "seconds": round(dt, 3),
            "host_cores_available": avail}


def bench_backward(args, w, mha):
    """One step = one mha_backward_train call (dq, dk, dv of sum(dout * out),
    the row term from the fp32 output of mha_forward_train) on inputs
    resident in device memory, the forward's outputs computed once
    beforehand. The same line carries mha_backward (row term from a pass over
    the keys, from mha_forward's outputs) as a sub-record. FLOPs: 10 * d_h per
    visible pair (the five products S, dP, dV, dQ, dK of 2 * d_h each)."""
    import torch
    import oracle
    from workloads import make_backward_inputs

    if w.dtype == torch.float32:
        raise SystemExit("the backward takes fp16 / bf16 inputs")
    K = args.steps if args.steps is not None else DEFAULT_STEPS.get(w.name, 20)
    W = args.warmup if args.warmup is not None else DEFAULT_WARMUP.get(w.name, 3)
    dev = torch.device("cuda:0")
    q, k, v, kl, dout = make_backward_inputs(w, args.seed, device=dev)
    kl_cpu = None if kl is None else kl.cpu()
    pairs = pair_count(w, kl_cpu)
    flops = 10 * w.D * pairs
    _, lse_t, out32 = mha.forward_train(q, k, v, causal=w.causal, key_len=kl)
    out, lse = mha.forward(q, k, v, causal=w.causal, key_len=kl)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty_like(lse)
    stream = torch.cuda.current_stream(dev)

    def step_train():
        mha.backward_train(q, k, v, out32, lse_t, dout, causal=w.causal, key_len=kl,
                           dq=dq, dk=dk, dv=dv, delta=delta, stream=stream)

    def step_exact():
        mha.backward(q, k, v, out, lse, dout, causal=w.causal, key_len=kl,
                     dq=dq, dk=dk, dv=dv, delta=delta, stream=stream)

    def timed(step):
        t_w = time.perf_counter()
        i = 0
        while i < W or time.perf_counter() - t_w < WARMUP_S:
            step()
            i += 1
            torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(stream)
        for _ in range(K):
            step()
        e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ev_ms = e0.elapsed_time(e1)
        return max(ev_ms, wall * 1e3) / K, ev_ms / K

    ms_exact, k_exact_ms = timed(step_exact)
    ms_per_step, k_avg_ms = timed(step_train)
    tag = dtype_tag(w.dtype)
    achieved = flops / (k_avg_ms * 1e-3) / 1e12
    peak = PEAK_MFMA_TFLOPS[tag]
    exact_achieved = flops / (k_exact_ms * 1e-3) / 1e12
    res = {
        "metric": "attention backward TFLOP/s (dq, dk, dv; 10*d_h flops per visible pair) "
                  "and % of MI355X MFMA roofline",
        "value": round(flops / (ms_per_step * 1e-3) / 1e12, 4),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": tag, "data": "synthetic",
        "config": {"workload": w.name, "pass": "backward", "B": w.B, "H": w.H,
                   "H_kv": w.H_kv or w.H, "S": w.S,
                   "d_h": w.D, "causal": w.causal,
                   "key_len": (None if w.key_len is None else list(w.key_len)), "seed": args.seed,
                   "entry_point": "mha_backward_train (inputs from mha_forward_train: out32, lse)",
                   "kernels": "row term dout . out32, then dq and dk/dv in one launch",
                   "parallelism": "single GPU"},
        "roofline": {
            "bound": "mfma", "achieved": round(achieved, 3), "peak": peak, "unit": "TFLOP/s",
            "frac": round(achieved / peak, 5),
            "traffic": stored_traffic(w.name, kernel_source_hash(BWD_SOURCES)),
            "kernel_avg_us": round(k_avg_ms * 1e3, 3),
            "kernel_timing": "HIP events around the timed region / %d backward calls "
                             "(all kernels of a call)" % K,
            "algorithmic_flops": flops, "kernel_source_hash": kernel_source_hash(BWD_SOURCES),
        },
        "flops_per_step": flops, "visible_pairs": pairs,
        "subrecords": {"mha_backward": {
            "entry_point": "mha_backward (inputs from mha_forward: out, lse)",
            "kernels": "row-term pass over the keys, then dq and dk/dv in one launch",
            "value": round(flops / (ms_exact * 1e-3) / 1e12, 4), "unit": "TFLOP/s",
            "ms_per_step": round(ms_exact, 6), "kernel_avg_us": round(k_exact_ms * 1e3, 3),
            "achieved": round(exact_achieved, 3), "frac": round(exact_achieved / peak, 5)}},
    }
    if not args.no_cpu_baseline:
        # the float64 oracle's backward on the whole workload
        avail = len(os.sched_getaffinity(0))
        try:
            from threadpoolctl import threadpool_info
            blas = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        except Exception:
            blas = 1
        qc, kc, vc, dc = (t.cpu() for t in (q, k, v, dout))
        if w.H_kv and w.H_kv != w.H:  # the oracle's heads: key / value heads repeated per group
            kc, vc = (t.repeat_interleave(w.H // w.H_kv, dim=1) for t in (kc, vc))
        reps = 0
        t0 = time.perf_counter()
        while True:  # the whole workload, repeated until about 12 s have passed
            oracle.attention_backward(qc, kc, vc, dc, causal=w.causal, key_len=kl_cpu)
            reps += 1
            dt = time.perf_counter() - t0
            if dt > 12.0:
                break
        sample_flops = reps * flops
        res["cpu_baseline"] = {"value": sample_flops / dt / 1e12, "unit": "TFLOP/s",
                               "cores": blas, "kind": "oracle",
                               "sample": f"whole workload, repeated x{reps}",
                               "seconds": round(dt, 3), "host_cores_available": avail}
    return res


def bench_qkv(args, w, mha):
    """One step = one mha_qkv_attention call: the QKV projection of x
    [B, S, d_model] and attention on its head slices, inputs resident in
    device memory. FLOPs: 6 S d_model^2 per batch element for the projection
    (x W_qkv over every row, as the definition states it) plus 4 d_h per
    visible pair for attention. Algorithmic bytes: x, W_qkv, b_qkv and the
    key lengths read once, out and lse written once."""
    import torch
    import oracle
    from workloads import make_qkv_inputs

    K = args.steps if args.steps is not None else DEFAULT_STEPS[w.name]
    W = args.warmup if args.warmup is not None else DEFAULT_WARMUP[w.name]
    dev = torch.device("cuda:0")
    tag = dtype_tag(w.dtype)
    esize = torch.tensor([], dtype=w.dtype).element_size()
    x, wq, bq, kl = make_qkv_inputs(w, args.seed, device=dev)
    kl_cpu = None if kl is None else kl.cpu()
    D = w.H * w.D
    pairs = pair_count(w, kl_cpu)
    flops = 6 * w.B * w.S * D * D + 4 * w.D * pairs
    nbytes = (2 * w.B * w.S * D + 3 * D * D + 3 * D) * esize + 4 * w.B * w.H * w.S \
        + (0 if kl is None else 4 * w.B)
    nsets = 1 if nbytes >= MALL_BYTES else max(3, min(8, math.ceil(2 * MALL_BYTES / max(nbytes, 1))))
    xs = [x] + [x.clone() for _ in range(nsets - 1)]
    outs = [(torch.empty_like(x), torch.empty((w.B, w.H, w.S), dtype=torch.float32, device=dev))
            for _ in range(nsets)]
    stream = torch.cuda.current_stream(dev)

    def step(i, s=None):
        o, l = outs[i % nsets]
        mha.qkv_attention(xs[i % nsets], wq, bq, n_heads=w.H, causal=w.causal, key_len=kl,
                          out=o, lse=l, stream=stream if s is None else s)

    t_w = time.perf_counter()
    i = 0
    while i < W or time.perf_counter() - t_w < WARMUP_S:
        step(i)
        i += 1
        torch.cuda.synchronize()

    def timed(run, n, st):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(st)
        run()
        e1.record(st)
        torch.cuda.synchronize()
        wall_s = time.perf_counter() - t0
        ev = e0.elapsed_time(e1)
        return max(ev, wall_s * 1e3) / n, ev

    G = args.graph if args.graph is not None else DEFAULT_GRAPH[w.name]
    g1, n_rep, g2 = graph_plan(K, G)
    graphs = capture_graphs(lambda i, s: step(i, s), (g1, g2), stream, dev)

    eager_ms, eager_ev = timed(lambda: [step(i) for i in range(K)], K, stream)
    ms_per_step, k_ev = eager_ms, eager_ev
    timing = "HIP events around the timed region / %d launches" % K
    if graphs:
        ms_per_step, k_ev = timed(lambda: replay_plan(graphs, n_rep), K, stream)
        timing = "HIP events around the timed graph replays / %d launches" % K
    k_avg_ms = k_ev / K

    # context: the same computation unfused -- a library GEMM for the
    # projection (torch addmm) and the attention kernel on the head views
    y = torch.empty((w.B, w.S, 3 * D), dtype=w.dtype, device=dev)
    uo = torch.empty((w.B, w.S, w.H, w.D), dtype=w.dtype, device=dev).transpose(1, 2)
    ul = torch.empty((w.B, w.H, w.S), dtype=torch.float32, device=dev)

    def unfused():
        torch.addmm(bq, x.view(-1, D), wq, out=y.view(-1, 3 * D))
        q, k, v = (t.view(w.B, w.S, w.H, w.D).transpose(1, 2) for t in y.split(D, dim=-1))
        mha.forward(q, k, v, causal=w.causal, key_len=kl, out=uo, lse=ul, stream=stream)

    for _ in range(3):
        unfused()
    n_u = max(1, min(K, 50))
    unfused_ms, _ = timed(lambda: [unfused() for _ in range(n_u)], n_u, stream)

    achieved = nbytes / (k_avg_ms * 1e-3) / 1e9
    mfma_achieved = flops / (k_avg_ms * 1e-3) / 1e12
    src_hash = kernel_source_hash(QKV_SOURCES)
    res = {
        "metric": "fused QKV projection + attention TFLOP/s (6 S d_model^2 projection flops per "
                  "batch element + 4 d_h per visible pair) and % of MI355X HBM roofline",
        "value": round(flops / (ms_per_step * 1e-3) / 1e12, 4),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": tag, "data": "synthetic",
        "config": {"workload": w.name, "pass": "qkv projection + forward", "B": w.B, "S": w.S,
                   "d_model": D, "H": w.H, "d_h": w.D, "causal": w.causal,
                   "key_len": (None if w.key_len is None else list(w.key_len)),
                   "seed": args.seed, "bias": True, "buffer_sets": nsets,
                   "parallelism": "single GPU",
                   "submission": submission(graphs, g1, n_rep, g2)},
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 3), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 5),
            "traffic": stored_traffic(w.name, src_hash),
            "kernel_avg_us": round(k_avg_ms * 1e3, 3), "kernel_timing": timing,
            "algorithmic_bytes": nbytes, "algorithmic_flops": flops,
            "mfma_tflops": round(mfma_achieved, 3),
            "mfma_frac": round(mfma_achieved / PEAK_MFMA_TFLOPS[tag], 5),
            "kernel_source_hash": src_hash,
        },
        "flops_per_step": flops, "visible_pairs": pairs,
        "eager_ms_per_step": round(eager_ms, 6),
        "unfused_ms_per_step": round(unfused_ms, 6),
        "unfused": "torch addmm (library GEMM) + mha_forward_strided on the head views, eager",
    }
    if not args.no_cpu_baseline:
        avail = len(os.sched_getaffinity(0))
        threads = max(1, min(16, avail))
        try:
            from threadpoolctl import threadpool_info
            blas = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        except Exception:
            blas = 1
        xc, wc, bc = x.cpu(), wq.cpu(), bq.cpu()
        # batch elements in chunks of 64 (in order, wrapping) until ~12 s
        chunk = min(64, w.B)
        done, t0, j = 0, time.perf_counter(), 0
        while True:
            idx = [(j + i) % w.B for i in range(chunk)]
            oracle.qkv_attention(xc[idx], wc, bc, w.H, causal=w.causal,
                                 key_len=None if kl_cpu is None else kl_cpu[idx], threads=threads)
            done += chunk
            j += chunk
            dt = time.perf_counter() - t0
            if dt > 12.0:
                break
        frac = done / w.B
        res["cpu_baseline"] = {"value": flops * frac / dt / 1e12, "unit": "TFLOP/s",
                               "cores": max(blas, threads), "kind": "oracle",
                               "sample": f"{done} batch elements (of {w.B}) in chunks of {chunk}",
                               "seconds": round(dt, 3), "host_cores_available": avail}
    return res


def copy_calibration(nbytes: int, reps: int):
    """A plain device copy of known size, for scaling the HBM byte counters."""
    import torch
    src = torch.empty(nbytes // 2, dtype=torch.float16, device="cuda").normal_()
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": nbytes, "bytes_written": nbytes, "reps": reps}))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default=None,
                    choices=["tiny", "launch", "bandwidth", "compute", "long", "bwd", "bwd_gqa",
                             "qkv_launch", "qkv_bandwidth", "qkv_heads8"],
                    help="default: the long-sequence forward (S=100000) with sub-records for the "
                         "bandwidth, compute and launch shapes; bwd for the backward")
    ap.add_argument("--pass", dest="which", default="fwd", choices=["fwd", "bwd"],
                    help="time the forward (default) or the backward (dq, dk, dv)")
    ap.add_argument("--variant", default="auto")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-subrecords", action="store_true",
                    help="time only the headline workload")
    ap.add_argument("--graph", type=int, default=None, metavar="G",
                    help="time steps as replays of a HIP graph of G calls (0 = eager)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MiB",
                    help="only run a plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU; --gpus must be 1",
                          "n_gpus_requested": args.gpus}), flush=True)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}), flush=True)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration << 20, 10)
        return

    import exact_attention_mha_amd as mha
    from workloads import WORKLOADS

    mha.load()  # raises if the HIP library is missing: there is no fallback
    headline = args.workload is None and args.which == "fwd"
    if args.workload is None:
        args.workload = "bwd" if args.which == "bwd" else HEADLINE
    w = WORKLOADS[args.workload]
    if args.which == "bwd":
        print(json.dumps(bench_backward(args, w, mha)), flush=True)
        return
    if w.name.startswith("qkv_"):
        print(json.dumps(bench_qkv(args, w, mha)), flush=True)
        return
    rec = bench_forward(w, mha, steps=args.steps, warmup=args.warmup, graph=args.graph,
                        variant=args.variant, seed=args.seed, cpu=not args.no_cpu_baseline)
    if headline and not args.no_subrecords:
        # the other forward regimes, each timed on its own kernel with its own
        # step count, roofline and CPU baseline, in the same line
        rec["subrecords"] = {}
        for name in SUBRECORDS:
            rec["subrecords"][name] = bench_forward(
                WORKLOADS[name], mha, steps=None, warmup=None, graph=None, variant="auto",
                seed=args.seed, cpu=not args.no_cpu_baseline, cpu_budget_s=SUB_CPU_BUDGET_S)
            print(f"# subrecord {name}: {rec['subrecords'][name]['roofline']['kernel_avg_us']} us "
                  f"per launch", file=sys.stderr, flush=True)
    print(json.dumps(rec), flush=True)


def graph_plan(steps: int, graph: int):
    """How K timed steps are submitted from HIP graphs of captured calls:
    (calls per graph, replays of it, calls in a second graph replayed once
    for the remainder). Always exactly `steps` calls in all; (0, 0, 0) for
    eager submission."""
    if graph <= 0 or steps <= 0:
        return 0, 0, 0
    g = min(graph, steps)
    return g, steps // g, steps % g


def capture_graphs(step, sizes, stream, dev):
    """Capture one HIP graph per nonzero size, each holding that many calls
    of step(i, capture_stream); every graph is replayed once, untimed."""
    import torch
    graphs = []
    if not sizes or sizes[0] <= 0:
        return graphs
    cap = torch.cuda.Stream(dev)
    for n in sizes:
        if n <= 0:
            continue
        gr = torch.cuda.CUDAGraph()
        cap.wait_stream(stream)
        with torch.cuda.stream(cap):
            with torch.cuda.graph(gr, stream=cap):
                for i in range(n):
                    step(i, cap)
        stream.wait_stream(cap)
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        graphs.append(gr)
    return graphs


def replay_plan(graphs, n_rep):
    for _ in range(n_rep):
        graphs[0].replay()
    if len(graphs) > 1:
        graphs[1].replay()


def submission(graphs, g1, n_rep, g2):
    if not graphs:
        return "eager"
    return f"hip graphs: {n_rep} replays of {g1} calls" + (f" + 1 of {g2}" if g2 else "")


def bench_forward(w, mha, *, steps=None, warmup=None, graph=None, variant="auto", seed=0, cpu=True,
                  cpu_budget_s=12.0):
    """One forward workload: K timed launches of the library's kernel on
    inputs resident in device memory. Returns the JSON record."""
    import torch
    from workloads import make_inputs

    K = steps if steps is not None else DEFAULT_STEPS[w.name]
    W = warmup if warmup is not None else DEFAULT_WARMUP[w.name]
    if K < 1:
        raise SystemExit("--steps must be at least 1")
    dev = torch.device("cuda:0")
    tag = dtype_tag(w.dtype)
    esize = torch.tensor([], dtype=w.dtype).element_size()

    q, k, v, kl = make_inputs(w, seed, device=dev)
    kl_cpu = None if kl is None else kl.cpu()
    pairs = pair_count(w, kl_cpu)
    flops = 4 * w.D * pairs
    conv_flops = 4 * w.B * w.H * w.S * w.S * w.D * (0.5 if w.causal else 1.0)
    nbytes = algorithmic_bytes(w, kl_cpu, esize)

    # rotate over several buffer sets when the working set would sit in the
    # 256 MB MALL, so repeated launches do not read warm inputs
    nsets = 1 if nbytes >= MALL_BYTES else max(3, min(8, math.ceil(2 * MALL_BYTES / max(nbytes, 1))))
    sets = [(q, k, v)]
    for _ in range(nsets - 1):
        sets.append((q.clone(), k.clone(), v.clone()))
    outs = [(torch.empty_like(q), torch.empty((w.B, w.H, w.S), dtype=torch.float32, device=dev))
            for _ in range(nsets)]
    stream = torch.cuda.current_stream(dev)
    variant_name = mha.select_variant(w.B, w.H, w.S, w.D, w.causal, w.dtype) \
        if variant == "auto" else variant

    def step(i, s=None):
        qq, kk, vv = sets[i % nsets]
        o, l = outs[i % nsets]
        mha.forward(qq, kk, vv, causal=w.causal, key_len=kl, out=o, lse=l,
                    variant=variant, stream=stream if s is None else s)

    # untimed warm-up: W steps, and at least WARMUP_S seconds of them, so the
    # GPU clock has ramped up before the timed region
    t_w = time.perf_counter()
    i = 0
    while i < W or time.perf_counter() - t_w < WARMUP_S:
        step(i)
        i += 1
        torch.cuda.synchronize()  # the clock check measures finished work

    def timed(run, n):
        """HIP events (on the kernel's stream) and the host wall clock around
        `run`: (ms per step by the larger of the two, event ms, wall s)."""
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(stream)
        run()
        e1.record(stream)
        torch.cuda.synchronize()
        wall_s = time.perf_counter() - t0
        ev = e0.elapsed_time(e1)
        return max(ev, wall_s * 1e3) / n, ev, wall_s

    def eager():
        for i in range(K):
            step(i)

    G = graph if graph is not None else DEFAULT_GRAPH[w.name]
    g1, n_rep, g2 = graph_plan(K, G)
    graphs = capture_graphs(step, (g1, g2), stream, dev)

    # ---- timed region: K back-to-back steps, eager; then, for the
    # launch-bound shapes, the same K calls submitted as graph replays
    eager_ms, eager_ev_ms, wall = timed(eager, K)
    ms_per_step = eager_ms
    if graphs:
        ms_per_step, graph_ev_ms, _ = timed(lambda: replay_plan(graphs, n_rep), K)

    # ---- kernel duration: HIP events on the kernel's stream around the timed
    # region, divided by the launches in it (one launch per step). Launches
    # run back to back, so this bounds the kernel's own duration from above
    # by the small gaps between them; an event pair around each single launch
    # would add its own marker and dispatch overhead instead.
    if graphs:
        k_avg_ms = graph_ev_ms / K
        kernel_timing = "HIP events around the timed graph replays / %d launches" % K
    else:
        k_avg_ms = eager_ev_ms / K
        kernel_timing = "HIP events around the timed region / %d launches" % K

    bound = BOUND[w.name]
    if bound == "hbm":
        achieved, peak, unit = nbytes / (k_avg_ms * 1e-3) / 1e9, PEAK_HBM_GBS, "GB/s"
    else:
        achieved, peak, unit = flops / (k_avg_ms * 1e-3) / 1e12, PEAK_MFMA_TFLOPS[tag], "TFLOP/s"
    src_hash = kernel_source_hash()
    traffic = stored_traffic(w.name, src_hash)

    value = flops / (ms_per_step * 1e-3) / 1e12
    res = {
        "metric": "attention TFLOP/s (causal-adjusted) and % of MI355X MFMA/HBM roofline",
        "value": round(value, 4),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": tag,
        "data": "synthetic",
        "config": {
            "workload": w.name, "B": w.B, "H": w.H, "S": w.S, "d_h": w.D, "causal": w.causal,
            "key_len": (None if w.key_len is None else list(w.key_len)), "seed": seed,
            "variant": variant_name, "buffer_sets": nsets, "parallelism": "single GPU",
            "submission": submission(graphs, g1, n_rep, g2),
        },
        "roofline": {
            "bound": bound, "achieved": round(achieved, 3), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 5), "traffic": traffic,
            "kernel_avg_us": round(k_avg_ms * 1e3, 3),
            "algorithmic_bytes": nbytes, "algorithmic_flops": flops,
            "kernel_source_hash": src_hash, "kernel_timing": kernel_timing,
        },
        "flops_per_step": flops,
        "conventional_causal_adjusted_flops": conv_flops,
        "visible_pairs": pairs,
        "hbm_gbs_per_step": round(nbytes / (ms_per_step * 1e-3) / 1e9, 3),
        "eager_ms_per_step": round(eager_ms, 6),
    }
    if bound == "mfma":
        res["roofline"]["hbm_gbs"] = round(nbytes / (k_avg_ms * 1e-3) / 1e9, 3)
    else:
        res["roofline"]["mfma_tflops"] = round(flops / (k_avg_ms * 1e-3) / 1e12, 3)
    if cpu:
        res["cpu_baseline"] = cpu_baseline(w, q, k, v, kl, 4 * w.D, budget_s=cpu_budget_s)
    del sets, outs, q, k, v
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


if __name__ == "__main__":
    main()
