#!/usr/bin/env python3
"""Benchmark of the structured-sparse plus low-rank linear layer on one MI355X.

A step is one pass of the hot path over one batch of seeded synthetic input.  By default it is
the OPT-13B-shaped MLP training step (hidden 5120, FFN 20480, T = 8192 tokens, both layers 2:4
bf16 with fp32 accumulation, rank-128 adapters), both layers chained:

    per layer: compress(W) + double_prune (one pass, in the streaming layout)
    fc1 forward (U1, Y1) -> fc2 forward on Y1 (U2, Y2)
        -> fc2 backward on dY2 (dU2, dX2, dB2, dA2) -> fc1 backward on dX2 (dU1, dX1, dB1, dA1)

Re-compressing every step mirrors a training loop that refreshes both compressed forms after each
optimizer update (SLoPe paperlayer summary §2.3).  The step is captured once in a HIP graph and
replayed.  Prints ONE JSON line with the throughput (dense-equivalent TFLOP/s), the speedup over
the dense bf16 GEMMs of the same chain (hipBLASLt through torch, same protocol), the roofline of
the dominant kernel (the 2:4 SpMM, timed live with HIP events around each launch alone), the
distribution of per-replay times, the smaller workloads as extras, and the CPU oracle timed on a
bounded sample as a reported baseline.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload opt13b_mlp]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "sparse+LoRA linear dense-equiv TFLOP/s & GB/s; speedup vs dense bf16 GEMM"
PEAK_BF16_FLOPS = 2.5e15   # MI355X dense bf16 MFMA (published); 2:4 work is priced as stored flops
PEAK_HBM_BPS = 8.0e12      # MI355X HBM3E (published)
PEAK_FP32_VALU = 157.3e12  # MI355X fp32 vector (published)

# Bytes between L2 and the fabric per launch (an upper bound on HBM bytes: the Infinity Cache may
# serve part of them) from rocprofv3 --pmc runs of `bench.py --loop <call>`
# (profiles/opt13b_mlp_spmm24_traffic.md, profiles/opt350m_fc1_spmm24_traffic.md,
# profiles/opt66b_ffn_decode_traffic.md).  Calibration: on gfx950 every read request counted by
# TCC_EA0_RDREQ moves a 128-byte line (TCC_BUBBLE and RDREQ_32B stay 0), so FETCH_SIZE, whose
# formula prices these at 64 bytes, reads half of a plain 256 MiB read or copy: FETCH_SIZE x 2.0,
# WRITE_SIZE x 1.0.  Keyed by the kernel configuration the planner picks for that call; a key
# missing here (kernel changed since the counters were taken) reports null.
TRAFFIC_BYTES = {
    "opt350m_fc1/2:4/canonical/spmm24_bwd/k_spmm24_pipe<2,1,2,2,4,16>": 27366.7 * 1024 * 2.0 + 4352.0 * 1024,
    "opt350m_fc1/2:4/canonical/spmm24_fwd/k_spmm24_q<4,4,4,2,3,8,16>": 13840.2 * 1024 * 2.0 + 16512.0 * 1024,
    # chained OPT-13B MLP step, streaming layout: mean per launch of the four 256x256 SpMM
    # products (profiles/opt13b_mlp_spmm24_traffic.md: TCC_EA0_RDREQ x 128 B + TCC_EA0_WRREQ x
    # 64 B, which equal FETCH_SIZE x 2.0 + WRITE_SIZE x 1.0 on gfx950)
    "opt13b_mlp/streaming/spmm24/k_spmm24_q<4, 8, 4, 2, 3, 4, 0, false, true, false>":
        18336572 * 128 + 3809929 * 64,
    # streaming layout (sra_nm_tile), 48-row workgroups of four waves, non-temporal weight loads
    # (profiles/opt66b_ffn_decode_traffic.md: read requests x 128 B + 64-byte and 32-byte writes)
    "opt66b_ffn_decode/T16/streaming/k_decode24<3>": 3042927 * 128 + 12288 * 64 + 12289 * 32,
    "opt66b_ffn_decode/T1/streaming/k_decode24<3>": 3025411 * 128 + 768 * 64 + 768 * 32,
    # the same weight at 2:8 on its streaming layout, k_decode28<9, 1, 256, 1, true>
    # (profiles/opt66b_ffn_decode_2_8_traffic.md)
    "opt66b_ffn_decode/T16/streaming/k_decode28<9,1>": 1725038 * 128 + 16384 * 64 + 4096 * 32,
    "opt66b_ffn_decode/T1/streaming/k_decode28<9,1>": 1711224 * 128 + 1024 * 64 + 256 * 32,
}


# The 256x256 SMFMAC SpMM instantiation the planner picks for all four products of the OPT-13B
# MLP step (fc1 Y, fc2 Y, fc2 dX, fc1 dX), by weight layout.
SPMM_MLP_KERNELS = {"streaming": "k_spmm24_q<4, 8, 4, 2, 3, 4, 0, false, true, false>",
                    "canonical": "k_spmm24_q<4, 8, 4, 2, 3, 4, 0, false, false, false>"}
ENGINE_EVAL_WHAT = {
    "2:4": "2:4 products on SMFMAC (the default) against the same pipeline with each weight fragment "
           "expanded to dense bf16 for dense MFMA",
    "2:8": "2:8 products on SMFMAC with the weight rewritten as 2:4 per call (the default above 16 "
           "tokens: every four columns of a 2:8 row hold at most two kept entries) against the 2:8 "
           "fragments expanded to dense bf16 for dense MFMA"}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="opt13b_mlp",
                    choices=["opt350m_fc1", "opt13b_fc1", "opt13b_fc2", "opt13b_mlp", "ffi90_4096",
                             "opt66b_ffn_decode", "squash_opt350m_fc2"])
    ap.add_argument("--decode-t", type=int, default=16, help="tokens for the decode workload")
    ap.add_argument("--decode-layout", choices=["streaming", "canonical"], default="streaming",
                    help="weight layout of the decode forward (streaming = sra_nm_tile)")
    ap.add_argument("--nm", choices=["2:4", "1:2", "2:8"], default="2:4",
                    help="N:M pattern of the training step's weight (1:2 runs on the 2:4 kernels, "
                         "2:8 on them too, rewritten as 2:4 per call)")
    ap.add_argument("--layout", choices=["canonical", "streaming"], default=None,
                    help="weight layout of the training step (streaming = sra_compress_pair_tiled); "
                         "default: streaming for opt13b_*, canonical otherwise")
    ap.add_argument("--no-graph", action="store_true", help="time eager calls instead of a graph")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of CPU oracle sampling")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--loop", choices=["spmm_fwd", "spmm_bwd", "decode", "copy", "read", "mlp"],
                    default=None,
                    help="run one call of the default workload --steps times and exit (for "
                         "rocprofv3 counter runs); 'copy' copies 256 MiB and 'read' sums 256 MiB "
                         "(counter calibration); "
                         "'mlp' runs the chained OPT-13B MLP step's calls")
    ap.add_argument("--no-ffi", action="store_true",
                    help="skip the fixed fan-in (90% sparse) layer measured beside the main line")
    ap.add_argument("--no-small", action="store_true",
                    help="skip the OPT-350M fc1 step measured beside the headline MLP step")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the OPT-66B decode measurements appended to the training-step line")
    args = ap.parse_args()
    if args.layout is None:
        args.layout = "streaming" if args.workload.startswith("opt13b") else "canonical"
    return args


# ----------------------------------------------------------------------------- work / bytes model

def step_model(wl, T, with_bwd=True, with_compress=True):
    """Dense-equivalent flops, algorithmic (stored) flops and algorithmic HBM bytes of one step."""
    K, N, r, e = wl.K, wl.N, wl.r, 2
    if wl.fmt == "ffi":
        w_bytes = N * wl.ffi_k * (e + 2)             # ELL values + int16 columns
        sparse_macs = T * N * wl.ffi_k
    else:
        w_bytes = N * K // 2 * e + N * K // 8        # stored values + 2-bit metadata
        sparse_macs = T * N * K // 2
    dense_eq = 2 * T * N * K + 2 * T * r * (K + N)  # forward
    algo = 2 * sparse_macs + 2 * T * r * (K + N)
    bytes_ = T * K * e + w_bytes + (r * K + N * r) * e + T * N * e + T * r * 4
    if with_bwd:
        dense_eq += 2 * T * N * K + 4 * T * r * (N + K)
        algo += 2 * sparse_macs + 4 * T * r * (N + K)
        bytes_ += T * N * e + T * K * e + w_bytes + T * r * 4 + (r * K + N * r) * e + T * K * e \
            + (r * K + N * r) * 4
    if with_compress and wl.fmt == "nm":
        bytes_ += N * K * e + w_bytes                # compress: read W, write Ws
        bytes_ += 2 * w_bytes                        # double prune: read Ws, write P
    return dense_eq, algo, bytes_


# ----------------------------------------------------------------------------- GPU timing helpers

def time_graph(fn, steps, warmup, use_graph=True, dist=None):
    """Wall-clock ms per call of fn over `steps` calls (graph replays), sync on both sides.

    With a dict as ``dist``, a second timed pass records a HIP event after every replay on the
    current stream and fills ``dist`` with the mean, median, p10 and p90 of the per-replay times."""
    import torch
    if use_graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(3):
                fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        run = g.replay
    else:
        run = fn
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        run()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    if dist is not None:
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        ev[0].record()
        for i in range(steps):
            run()
            ev[i + 1].record()
        torch.cuda.synchronize()
        dist.update(replay_stats([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]))
    return ms


def replay_stats(ts):
    """mean, median, p10, p90 (ms) of a list of per-replay times."""
    import numpy as np
    a = np.asarray(ts, dtype=np.float64)
    return {"n": int(a.size), "mean_ms": round(float(a.mean()), 5),
            "median_ms": round(float(np.median(a)), 5),
            "p10_ms": round(float(np.percentile(a, 10)), 5),
            "p90_ms": round(float(np.percentile(a, 90)), 5)}


def time_kernel(which, call, reps):
    """Average duration (ms) of one kernel class inside `call`, from HIP events placed around
    that kernel alone by the library's profiling hook, on the stream it is launched on."""
    import torch

    import sparse_rank_adapter_amd as sra
    pairs = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        sra.time_next_kernel(which, e0, e1)
        call()
        pairs.append((e0, e1))
    torch.cuda.synchronize()
    ts = sorted(a.elapsed_time(b) for a, b in pairs)
    return sum(ts) / len(ts)


def time_kernel_dist(which, call, reps):
    """time_kernel, returning the per-launch times as well (mean, distribution)."""
    import torch

    import sparse_rank_adapter_amd as sra
    pairs = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        sra.time_next_kernel(which, e0, e1)
        call()
        pairs.append((e0, e1))
    torch.cuda.synchronize()
    ts = [a.elapsed_time(b) for a, b in pairs]
    return sum(ts) / len(ts), ts


# ----------------------------------------------------------------------------- CPU oracle baseline

def host_info():
    """Host CPU facts for the CPU baseline: model, logical CPUs, the process's CPU share and the
    threads the oracle's numpy BLAS actually runs."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # threadpoolctl missing: report the host's view
        threads = os.cpu_count() or 1
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count() or 1
    return {"cpu_model": model, "nproc": os.cpu_count(), "affinity": affinity,
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS"), "blas_threads": int(threads)}


def _oracle_layer_step(X, W, A, B, dY, K):
    """compress + double prune + forward + backward of one layer with the oracle (float64)."""
    import numpy as np

    from oracle import layer as olayer
    from oracle import nm as onm
    v, m, mask1 = onm.compress(W, 2, 4)
    _, _, _, Wdp = onm.double_prune(v, m, 2, 4, K)
    Y, U = olayer.forward(X, np.where(mask1, W, 0.0), A, B)
    olayer.backward(dY, X, Wdp, A, B, U)


def cpu_baseline(wl, inp, budget_s, dense_eq_per_step, threads=None):
    """The oracle (float64 numpy) on full steps of a single-layer workload within a time budget;
    ``threads`` limits numpy's BLAS pool (None: as the process runs it)."""
    import contextlib

    import numpy as np
    ctx = contextlib.nullcontext()
    if threads is not None:
        from threadpoolctl import threadpool_limits
        ctx = threadpool_limits(threads)
    f64 = lambda t: t.detach().float().cpu().numpy().astype(np.float64)  # noqa: E731
    X, W, A, B, dY = (f64(inp[k]) for k in ("X", "W", "A", "B", "dY"))
    reps, t_total = 0, 0.0
    with ctx:
        used = host_info()["blas_threads"]
        while t_total < budget_s or reps == 0:
            t0 = time.perf_counter()
            _oracle_layer_step(X, W, A, B, dY, wl.K)
            t_total += time.perf_counter() - t0
            reps += 1
            if reps >= 20000:
                break
    return {"value": round(dense_eq_per_step * reps / t_total / 1e12, 5), "unit": "TFLOP/s",
            "cores": int(used), "kind": "oracle",
            "sample": f"{reps} full {wl.name} steps (compress + double_prune + fwd + bwd) in float64 "
                      f"numpy, {t_total:.2f} s"}


def cpu_baseline_mlp(i1, i2, budget_s, ffn_slice=1280):
    """The oracle on a bounded sample of the chained OPT-13B MLP step: the chain restricted to the
    FFN features [0, ffn_slice) (fc1's first output rows, fc2's first input columns; 1/16 of the
    20480 at the default), all 8192 tokens.  Every part of the step (both weights' compress and
    double prune, the four products and the adapter terms) is linear in the FFN width, so the
    sample is 1/16 of the step's work; its rate is reported on its own dense-equivalent flops."""
    import numpy as np

    from oracle import layer as olayer
    from oracle import nm as onm
    from sra_inputs import WORKLOADS
    f64 = lambda t: t.detach().float().cpu().numpy().astype(np.float64)  # noqa: E731
    X, A1, dY2, B2 = f64(i1["X"]), f64(i1["A"]), f64(i2["dY"]), f64(i2["B"])
    W1 = f64(i1["W"][:ffn_slice])
    B1 = f64(i1["B"][:ffn_slice])
    W2 = f64(i2["W"][:, :ffn_slice].contiguous())
    A2 = f64(i2["A"][:, :ffn_slice].contiguous())
    w1, w2 = WORKLOADS["opt13b_fc1"], WORKLOADS["opt13b_fc2"]
    T, H = X.shape
    sub1 = type(w1)("fc1_slice", T=T, K=H, N=ffn_slice, r=w1.r, dtype="bf16", fmt="nm")
    sub2 = type(w2)("fc2_slice", T=T, K=ffn_slice, N=H, r=w2.r, dtype="bf16", fmt="nm")
    flops = step_model(sub1, T, with_compress=False)[0] + step_model(sub2, T, with_compress=False)[0]
    reps, t_total = 0, 0.0
    while t_total < budget_s or reps == 0:
        t0 = time.perf_counter()
        v1, m1, mask1 = onm.compress(W1, 2, 4)
        _, _, _, Wdp1 = onm.double_prune(v1, m1, 2, 4, H)
        v2, m2, mask2 = onm.compress(W2, 2, 4)
        _, _, _, Wdp2 = onm.double_prune(v2, m2, 2, 4, ffn_slice)
        Y1, U1 = olayer.forward(X, np.where(mask1, W1, 0.0), A1, B1)
        _, U2 = olayer.forward(Y1, np.where(mask2, W2, 0.0), A2, B2)
        g2 = olayer.backward(dY2, Y1, Wdp2, A2, B2, U2)
        olayer.backward(g2["dX"], X, Wdp1, A1, B1, U1)
        t_total += time.perf_counter() - t0
        reps += 1
    info = host_info()
    return {"value": round(flops * reps / t_total / 1e12, 5), "unit": "TFLOP/s",
            "cores": info["blas_threads"], "kind": "oracle",
            "sample": f"{reps} x the chained opt13b_mlp step restricted to FFN features "
                      f"[0, {ffn_slice}) of 20480 (1/{20480 // ffn_slice} of every part: both "
                      f"weights' compress + double_prune on their slices, fc1 -> fc2 -> fc2 bwd -> "
                      f"fc1 bwd over all {T} tokens) in float64 numpy, {t_total:.1f} s; rate on "
                      f"the sample's own dense-equivalent flops",
            "host": info}


def cpu_one_thread(budget_s=4.0):
    """1-thread oracle figures on the tiny fp32 workload and the OPT-350M fc1 step."""
    from sra_inputs import WORKLOADS, layer_inputs
    out = {}
    for name, b in (("tiny_f32", 1.0), ("opt350m_fc1", budget_s)):
        wl = WORKLOADS[name]
        inp = layer_inputs(wl, seed=0)
        dense_eq = step_model(wl, wl.T, with_compress=False)[0]
        out[name] = cpu_baseline(wl, inp, b, dense_eq, threads=1)
    return out


# ----------------------------------------------------------------------------- workloads

def bench_nm_layer(args, wl):
    import torch

    import sparse_rank_adapter_amd as sra
    from sparse_rank_adapter_amd._abi import SRA_KERNEL_COMPRESS, SRA_KERNEL_DOUBLE_PRUNE, SRA_KERNEL_SPMM24
    from sra_inputs import layer_inputs

    dev = torch.device("cuda:0")
    inp = layer_inputs(wl, seed=0)
    X, W, A, B, dY = (inp[k].to(dev) for k in ("X", "W", "A", "B", "dY"))
    T, r = wl.T, wl.r
    tiled = args.layout == "streaming"
    n_, m_ = (int(x) for x in args.nm.split(":"))
    if tiled and (n_, m_) != (2, 4):
        raise SystemExit("the streaming layout is 2:4 only")
    if tiled:
        S, P = sra.compress_pair_tiled(W)
        pair = lambda: sra.compress_pair_tiled(W, out=(S, P))  # noqa: E731
    else:
        S = sra.compress(W, n_, m_)
        P = sra.double_prune(S)
        if m_ == 8:  # no one-pass pair kernel for 2:8
            def pair():
                sra.compress(W, n_, m_, out=S)
                sra.double_prune(S, out=P)
        else:
            pair = lambda: sra.compress_pair(W, n_, m_, out=(S, P))  # noqa: E731
    Y = torch.empty((T, wl.N), dtype=X.dtype, device=dev)
    U = torch.empty((T, r), dtype=torch.float32, device=dev)

    def ws_max(fn, M):  # a workspace large enough for both engines
        with sra.tuned(engine="dense_mfma"):
            b = fn(M, T, r)
        return max(1, b, fn(M, T, r))
    ws_f = torch.empty(ws_max(sra.fwd_workspace, S), dtype=torch.uint8, device=dev)
    ws_b = torch.empty(ws_max(sra.bwd_workspace, P), dtype=torch.uint8, device=dev)
    grads = {"dX": torch.empty((T, wl.K), dtype=X.dtype, device=dev),
             "dA": torch.empty((r, wl.K), dtype=torch.float32, device=dev),
             "dB": torch.empty((wl.N, r), dtype=torch.float32, device=dev)}

    def fwd():
        sra.sparse_lora_fwd(S, X, A, B, Y=Y, U=U, ws=ws_f)

    def bwd():
        sra.sparse_lora_bwd(P, dY, X, U, A, B, ws=ws_b, out=grads)

    def step():
        pair()  # compress and double prune in one pass over W
        fwd()
        bwd()

    graph = not args.no_graph
    dist = {}
    ms = time_graph(step, args.steps, args.warmup, graph, dist=dist)
    ms_fwd = time_graph(fwd, args.steps, args.warmup, graph)
    ms_bwd = time_graph(bwd, args.steps, args.warmup, graph)
    ms_cmp = time_graph(pair, args.steps, args.warmup, graph)
    # dense bf16 baseline: the same layer's forward and input-gradient GEMMs (hipBLASLt)
    Wd = W.contiguous()
    d_fwd = time_graph(lambda: torch.nn.functional.linear(X, Wd), args.steps, args.warmup, graph)
    d_bwd = time_graph(lambda: torch.matmul(dY, Wd), args.steps, args.warmup, graph)
    # informational: the same layer done densely in torch (bf16 GEMMs for the weight and LoRA)
    Ac, Bc = A.contiguous(), B.contiguous()

    def dl_fwd():
        return torch.nn.functional.linear(X, Wd) + torch.nn.functional.linear(
            torch.nn.functional.linear(X, Ac), Bc)

    def dl_bwd():
        dUd = torch.matmul(dY, Bc)
        return (torch.matmul(dY, Wd) + torch.matmul(dUd, Ac), torch.matmul(dUd.t().contiguous(), X),
                torch.matmul(dY.t().contiguous(), torch.nn.functional.linear(X, Ac)))
    dl_f = time_graph(dl_fwd, args.steps, args.warmup, graph)
    dl_b = time_graph(dl_bwd, args.steps, args.warmup, graph)

    # per-kernel durations inside the real calls (eager, hook-armed)
    reps = max(10, args.steps)
    k_fwd = time_kernel(SRA_KERNEL_SPMM24, fwd, reps)
    k_bwd = time_kernel(SRA_KERNEL_SPMM24, lambda: sra.sparse_lora_bwd(P, dY, X, U, A, B, ws=ws_b, out=grads), reps)
    k_pair = time_kernel(SRA_KERNEL_COMPRESS, pair, reps)
    # the separate single passes exist for the canonical arrays only
    k_cmp = None if tiled else time_kernel(SRA_KERNEL_COMPRESS, lambda: sra.compress(W, n_, m_, out=S), reps)
    k_dp = None if tiled else time_kernel(SRA_KERNEL_DOUBLE_PRUNE, lambda: sra.double_prune(S, out=P), reps)

    # masked weight gradient of the sparse weight (sparse training's weight update input):
    # dWs = (dY^T X) o mask1 in Ws's value order, against the dense dY^T X GEMM
    wg = None
    if not tiled and m_ != 8:
        from sparse_rank_adapter_amd._abi import SRA_KERNEL_WEIGHT_GRAD
        gW = torch.empty((wl.N, wl.K // 2), dtype=X.dtype, device=dev)
        k_wg = time_kernel(SRA_KERNEL_WEIGHT_GRAD, lambda: sra.masked_weight_grad(S, dY, X, out=gW), reps)
        dYt = dY.t().contiguous()
        d_wg = time_graph(lambda: torch.matmul(dYt, X), args.steps, args.warmup, graph)
        wg_flops = 2 * T * wl.N * wl.K   # the dense block product the kernel performs
        wg = {"kernel_ms": round(k_wg, 5),
              "dense_block_tflops": round(wg_flops / (k_wg * 1e-3) / 1e12, 2),
              "frac_bf16_mfma": round(wg_flops / (k_wg * 1e-3) / PEAK_BF16_FLOPS, 4),
              "dense_dW_gemm_ms": round(d_wg, 5),
              "speedup_vs_dense_dW": round(d_wg / k_wg, 3)}

    ev = None
    if args.nm in ("2:4", "2:8"):
        # the same layer with its products on the dense-MFMA engine (expanded fragments)
        with sra.tuned(engine="dense_mfma"):
            e_fwd = time_graph(fwd, args.steps, args.warmup, graph)
            e_bwd = time_graph(bwd, args.steps, args.warmup, graph)
            ek_fwd = time_kernel(SRA_KERNEL_SPMM24, fwd, reps)
            ek_bwd = time_kernel(SRA_KERNEL_SPMM24, lambda: sra.sparse_lora_bwd(P, dY, X, U, A, B, ws=ws_b,
                                                                                out=grads), reps)
        ev = {"what": ENGINE_EVAL_WHAT[args.nm],
              "smfmac": {"fwd_ms": round(ms_fwd, 5), "bwd_ms": round(ms_bwd, 5),
                         "spmm_fwd_kernel_ms": round(k_fwd, 5), "spmm_bwd_kernel_ms": round(k_bwd, 5)},
              "dense_mfma": {"fwd_ms": round(e_fwd, 5), "bwd_ms": round(e_bwd, 5),
                             "spmm_fwd_kernel_ms": round(ek_fwd, 5), "spmm_bwd_kernel_ms": round(ek_bwd, 5)},
              "smfmac_speedup_fwd_bwd": round((e_fwd + e_bwd) / (ms_fwd + ms_bwd), 3)}

    dense_eq, algo, nbytes = step_model(wl, T)
    # dominant kernel: the slower of the two SpMM launches; algorithmic flops per launch are the
    # stored products plus the adapter epilogue (2 T N K n/m + 2 T r R)
    spmm_flops_fwd = 2 * T * wl.N * (wl.K * n_ // m_) + 2 * T * r * wl.N
    spmm_flops_bwd = 2 * T * wl.K * (wl.N * n_ // m_) + 2 * T * r * wl.K
    if k_bwd >= k_fwd:
        kname, kms, kflops = "k_spmm24 (backward dX = dY P^T + dU A)", k_bwd, spmm_flops_bwd
        tkey = f"{wl.name}/{args.nm}/{args.layout}/spmm24_bwd/k_spmm24_pipe<2,1,2,2,4,16>"
    else:
        kname, kms, kflops = "k_spmm24 (forward Y = X Ws^T + U B^T)", k_fwd, spmm_flops_fwd
        tkey = f"{wl.name}/{args.nm}/{args.layout}/spmm24_fwd/k_spmm24_q<4,4,4,2,3,8,16>"
    traffic = TRAFFIC_BYTES.get(tkey)
    achieved = kflops / (kms * 1e-3) / 1e12
    out = {
        "metric": METRIC,
        "value": round(dense_eq / (ms * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "T": T, "K": wl.K, "N": wl.N, "r": r, "sparsity": args.nm,
                   "layout": args.layout,
                   "step": "compress + double_prune (one pass) + fwd + bwd (dX, dA, dB)",
                   "graph": graph, "seed": 0},
        "replay_ms": dist,
        "gbps": round(nbytes / (ms * 1e-3) / 1e9, 1),
        # fwd + bwd against the dense layer's two GEMMs; compress and double prune are the
        # method's one-time setup (the mask is fixed) and are timed separately
        "speedup_vs_dense": round((d_fwd + d_bwd) / (ms_fwd + ms_bwd), 3),
        "speedup_step_incl_compress_vs_dense": round((d_fwd + d_bwd) / ms, 3),
        "speedup_vs_dense_lora": round((dl_f + dl_b) / (ms_fwd + ms_bwd), 3),
        "detail_ms": {"step": round(ms, 5), "fwd": round(ms_fwd, 5), "bwd": round(ms_bwd, 5),
                      "compress+double_prune": round(ms_cmp, 5), "dense_fwd_gemm": round(d_fwd, 5),
                      "dense_dx_gemm": round(d_bwd, 5), "dense_lora_fwd": round(dl_f, 5),
                      "dense_lora_bwd": round(dl_b, 5)},
        "speedup_fwd_vs_dense_fwd": round(d_fwd / ms_fwd, 3),
        "speedup_bwd_vs_dense_dx": round(d_bwd / ms_bwd, 3),
        "kernel_ms": {"spmm24_fwd": round(k_fwd, 5), "spmm24_bwd": round(k_bwd, 5),
                      "compress_pair": round(k_pair, 5),
                      "compress": None if k_cmp is None else round(k_cmp, 5),
                      "double_prune": None if k_dp is None else round(k_dp, 5)},
        "masked_weight_grad": wg,
        "engine_eval": ev,
        # Lemma 2.1's quantity on the GPU's own compressed forms: entries the second prune removed,
        # over all N K entries (Gaussian weights: every kept value is nonzero)
        "added_zeros_frac": None if tiled else round(
            (int((S.values != 0).sum()) - int((P.values != 0).sum())) / (wl.N * wl.K), 5),
        "roofline": {"kernel": kname, "bound": "mfma", "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_FLOPS / 1e12, "unit": "TFLOP/s",
                     "frac": round(achieved * 1e12 / PEAK_BF16_FLOPS, 4),
                     "traffic": round(traffic) if traffic else None},
    }
    return out, inp, dense_eq


def bench_mlp_chain(args, inputs=None, nm="2:4", engine_eval=True):
    """OPT-13B MLP step with both layers chained: fc1 forward on X, fc2 forward on fc1's Y, fc2
    backward on dY2, fc1 backward on fc2's dX (no activation between the layers), each layer's
    compress + double prune first; against the four dense GEMMs of the same chain.  nm = "2:8"
    runs both weights at 2:8 (canonical arrays; the products rewrite them as 2:4 for SMFMAC);
    engine_eval also times the same step with the products on the dense-MFMA engine (weight
    fragments expanded to dense bf16) beside the SMFMAC one.

    Returns (line, (i1, i2)) with the CPU inputs of both layers for the CPU baseline."""
    import torch

    import sparse_rank_adapter_amd as sra
    from sparse_rank_adapter_amd._abi import SRA_KERNEL_SPMM24
    from sra_inputs import WORKLOADS, layer_inputs

    dev = torch.device("cuda:0")
    w1, w2 = WORKLOADS["opt13b_fc1"], WORKLOADS["opt13b_fc2"]
    i1, i2 = inputs if inputs is not None else (layer_inputs(w1, seed=0, with_dy=False),
                                                layer_inputs(w2, seed=0))
    X, W1, A1, B1 = (i1[k].to(dev) for k in ("X", "W", "A", "B"))
    W2, A2, B2, dY2 = (i2[k].to(dev) for k in ("W", "A", "B", "dY"))
    T = w1.T
    n_, m_ = (int(x) for x in nm.split(":"))
    tiled = args.layout == "streaming" and nm == "2:4"
    layers = []

    def ws_max(fn, M):  # a workspace large enough for both engines
        with sra.tuned(engine="dense_mfma"):
            b = fn(M, T, r)
        return max(1, b, fn(M, T, r))
    for wl, W, A, B in ((w1, W1, A1, B1), (w2, W2, A2, B2)):
        if tiled:
            S, P = sra.compress_pair_tiled(W)
        elif nm == "2:4":
            S, P = sra.compress_pair(W)
        else:
            S = sra.compress(W, n_, m_)
            P = sra.double_prune(S)
        r = wl.r
        layers.append(dict(
            wl=wl, W=W, A=A, B=B, S=S, P=P,
            Y=torch.empty((T, wl.N), dtype=X.dtype, device=dev),
            U=torch.empty((T, r), dtype=torch.float32, device=dev),
            ws_f=torch.empty(ws_max(sra.fwd_workspace, S), dtype=torch.uint8, device=dev),
            ws_b=torch.empty(ws_max(sra.bwd_workspace, P), dtype=torch.uint8, device=dev),
            g={"dX": torch.empty((T, wl.K), dtype=X.dtype, device=dev),
               "dA": torch.empty((r, wl.K), dtype=torch.float32, device=dev),
               "dB": torch.empty((wl.N, r), dtype=torch.float32, device=dev)}))
    l1, l2 = layers

    def pairs():
        for L in layers:
            if tiled:
                sra.compress_pair_tiled(L["W"], out=(L["S"], L["P"]))
            elif nm == "2:4":
                sra.compress_pair(L["W"], out=(L["S"], L["P"]))
            else:
                sra.compress(L["W"], n_, m_, out=L["S"])
                sra.double_prune(L["S"], out=L["P"])

    def fwd1():
        sra.sparse_lora_fwd(l1["S"], X, l1["A"], l1["B"], Y=l1["Y"], U=l1["U"], ws=l1["ws_f"])

    def fwd2():
        sra.sparse_lora_fwd(l2["S"], l1["Y"], l2["A"], l2["B"], Y=l2["Y"], U=l2["U"], ws=l2["ws_f"])

    def bwd2():
        sra.sparse_lora_bwd(l2["P"], dY2, l1["Y"], l2["U"], l2["A"], l2["B"], ws=l2["ws_b"], out=l2["g"])

    def bwd1():
        sra.sparse_lora_bwd(l1["P"], l2["g"]["dX"], X, l1["U"], l1["A"], l1["B"], ws=l1["ws_b"],
                            out=l1["g"])

    def fwd():
        fwd1()
        fwd2()

    def bwd():
        bwd2()
        bwd1()

    def step():
        pairs()
        fwd()
        bwd()

    graph = not args.no_graph
    dist = {}
    ms = time_graph(step, args.steps, args.warmup, graph, dist=dist)
    ms_fwd = time_graph(fwd, args.steps, args.warmup, graph)
    ms_bwd = time_graph(bwd, args.steps, args.warmup, graph)
    ms_pairs = time_graph(pairs, args.steps, args.warmup, graph)
    W1d, W2d = W1.contiguous(), W2.contiguous()
    Y1d = torch.nn.functional.linear(X, W1d)
    dX2d = torch.matmul(dY2, W2d)
    d_dist = {}
    d_fwd = time_graph(lambda: (torch.nn.functional.linear(X, W1d), torch.nn.functional.linear(Y1d, W2d)),
                       args.steps, args.warmup, graph)
    d_bwd = time_graph(lambda: (torch.matmul(dY2, W2d), torch.matmul(dX2d, W1d)),
                       args.steps, args.warmup, graph)
    d_all = time_graph(lambda: (torch.nn.functional.linear(X, W1d), torch.nn.functional.linear(Y1d, W2d),
                                torch.matmul(dY2, W2d), torch.matmul(dX2d, W1d)),
                       args.steps, args.warmup, graph, dist=d_dist)

    # the dominant kernel: the 2:4 SpMM with the fused adapter epilogue, four launches per step
    # (fc1 Y, fc2 Y, fc2 dX, fc1 dX), each timed alone by the library's hook on its own stream.
    # Algorithmic flops per launch: stored-half products 2 T R (C/2) plus the epilogue 2 T r R.
    reps = max(10, args.steps)

    def spmm_launches():
        out = []
        for name, call, R, C in (("fc1_fwd", fwd1, w1.N, w1.K), ("fc2_fwd", fwd2, w2.N, w2.K),
                                 ("fc2_dx", bwd2, w2.K, w2.N), ("fc1_dx", bwd1, w1.K, w1.N)):
            mean, ts = time_kernel_dist(SRA_KERNEL_SPMM24, call, reps)
            fl = 2 * T * R * (C * n_ // m_) + 2 * T * w1.r * R   # stored products + epilogue
            fd = 2 * T * R * C + 2 * T * w1.r * R                 # the same on the dense weight
            out.append({"call": name, "rows": R, "reduction": C, "flops": fl,
                        "kernel_ms": round(mean, 5),
                        "kernel_median_ms": round(float(sorted(ts)[len(ts) // 2]), 5),
                        "tflops_stored": round(fl / (mean * 1e-3) / 1e12, 1),
                        "tflops_dense_eq": round(fd / (mean * 1e-3) / 1e12, 1)})
        return out
    launches = spmm_launches()
    k_flops = sum(L["flops"] for L in launches) / len(launches)
    k_ms = sum(L["kernel_ms"] for L in launches) / len(launches)
    achieved = k_flops / (k_ms * 1e-3) / 1e12
    kname = SPMM_MLP_KERNELS[args.layout] if nm == "2:4" else SPMM_MLP_KERNELS["canonical"]
    traffic = TRAFFIC_BYTES.get(f"opt13b_mlp/{args.layout}/spmm24/{kname}") if nm == "2:4" else None
    ev = None
    if engine_eval and nm in ("2:4", "2:8"):
        # the same step with the products on the dense-MFMA engine (graphs captured under it)
        with sra.tuned(engine="dense_mfma"):
            e_ms = time_graph(step, args.steps, args.warmup, graph)
            e_fwd = time_graph(fwd, args.steps, args.warmup, graph)
            e_bwd = time_graph(bwd, args.steps, args.warmup, graph)
            e_launches = spmm_launches()
        e_k = sum(L["kernel_ms"] for L in e_launches) / len(e_launches)
        ev = {"what": ENGINE_EVAL_WHAT[nm],
              "smfmac": {"step_ms": round(ms, 5), "fwd_ms": round(ms_fwd, 5), "bwd_ms": round(ms_bwd, 5),
                         "spmm_kernel_ms_mean": round(k_ms, 5)},
              "dense_mfma": {"step_ms": round(e_ms, 5), "fwd_ms": round(e_fwd, 5), "bwd_ms": round(e_bwd, 5),
                             "spmm_kernel_ms_mean": round(e_k, 5),
                             "spmm_launches": [{k: L[k] for k in ("call", "kernel_ms", "tflops_dense_eq")}
                                               for L in e_launches]},
              "smfmac_speedup_spmm": round(e_k / k_ms, 3),
              "smfmac_speedup_fwd_bwd": round((e_fwd + e_bwd) / (ms_fwd + ms_bwd), 3)}

    dense_eq = sum(step_model(L["wl"], T, with_compress=False)[0] for L in layers)
    line = {
        "metric": METRIC,
        "value": round(dense_eq / (ms * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "opt13b_mlp", "T": T, "hidden": w1.K, "ffn": w1.N, "r": w1.r,
                   "sparsity": nm, "layout": "streaming" if tiled else "canonical",
                   "step": "per layer compress + double_prune; fc1 fwd, fc2 fwd, fc2 bwd (dX, dA, dB), "
                           "fc1 bwd (dX, dA, dB)",
                   "graph": graph, "seed": 0},
        # per-replay HIP-event times of the timed step (a second pass of the same replays)
        "replay_ms": dist,
        # fwd + bwd of both layers against the chain's four dense GEMMs (X W1^T, Y1 W2^T, dY2 W2,
        # dX2 W1); compress and double prune are the method's setup and are timed apart
        "speedup_vs_dense": round((d_fwd + d_bwd) / (ms_fwd + ms_bwd), 3),
        "speedup_step_incl_compress_vs_dense": round((d_fwd + d_bwd) / ms, 3),
        "speedup_fwd_vs_dense_fwd": round(d_fwd / ms_fwd, 3),
        "speedup_bwd_vs_dense_dx": round(d_bwd / ms_bwd, 3),
        "detail_ms": {"step": round(ms, 5), "fwd": round(ms_fwd, 5), "bwd": round(ms_bwd, 5),
                      "compress+double_prune": round(ms_pairs, 5),
                      "dense_fwd_gemms": round(d_fwd, 5), "dense_dx_gemms": round(d_bwd, 5),
                      "dense_four_gemms": round(d_all, 5)},
        "dense_replay_ms": d_dist,
        "spmm_launches": launches,
        "roofline": {"kernel": f"{kname} (" + ("2:4" if nm == "2:4" else "2:8 rewritten as 2:4")
                               + " SpMM + adapter epilogue; mean of the four launches of a step)",
                     "bound": "mfma", "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_FLOPS / 1e12, "unit": "TFLOP/s",
                     "frac": round(achieved * 1e12 / PEAK_BF16_FLOPS, 4),
                     "traffic": round(traffic) if traffic else None,
                     "algorithmic_flops_per_launch": int(k_flops),
                     "kernel_ms": round(k_ms, 5)},
    }
    if ev:
        line["engine_eval"] = ev
    return line, (i1, i2)


def decode_bytes(wl, T, kernel_only=False, m=4):
    """Algorithmic HBM bytes of one decode forward call (or of the decode kernel alone: the
    down-projection U = X A^T reads A in its own launch, the kernel reads U instead), for a 2:4
    (m = 4) or 2:8 (m = 8) weight."""
    K, N, r, e = wl.K, wl.N, wl.r, 2
    w = N * K * 2 // m * e + N * K // 8                  # stored values + metadata (1 bit per entry)
    common = w + N * r * e + T * K * e + T * N * e      # + B, X, Y
    return common + (T * r * 4 if kernel_only else r * K * e)


def bench_decode(args, wl, Ts):
    """Forward at decode token counts on the streaming layout of the weight (sra_nm_tile), with
    the decode kernel on the canonical arrays timed beside it.  Two compressed copies of the
    weight (2 x 382 MB) are alternated so that the 256 MB Infinity Cache cannot serve a repeated
    read; the dense comparator alternates two dense copies the same way."""
    import torch

    import sparse_rank_adapter_amd as sra
    from sparse_rank_adapter_amd._abi import SRA_KERNEL_DECODE24
    from sra_inputs import layer_inputs

    dev = torch.device("cuda:0")
    inp = layer_inputs(wl, seed=0, T=max(Ts), with_dy=False)
    X, W, A, B = (inp[k].to(dev) for k in ("X", "W", "A", "B"))
    r = wl.r
    canon = (sra.compress(W), sra.compress(W))
    streaming = tuple(sra.nm_tile(S) for S in canon)
    nm28 = (sra.compress(W, 2, 8), sra.compress(W, 2, 8))
    nm28t = tuple(sra.nm_tile(S) for S in nm28)
    main, other = (streaming, canon) if args.decode_layout == "streaming" else (canon, streaming)
    dense = (W, W.clone())
    rows = []
    for T in Ts:
        Xt = X[:T].contiguous()
        Y = torch.empty((T, wl.N), dtype=X.dtype, device=dev)
        U = torch.empty((T, r), dtype=torch.float32, device=dev)
        ws = torch.empty(max(1, sra.fwd_workspace(canon[0], T, r)), dtype=torch.uint8, device=dev)

        def both():
            for S in main:
                sra.sparse_lora_fwd(S, Xt, A, B, Y=Y, U=U, ws=ws)

        def alternate(copies):
            flip = [0]

            def one():
                S = copies[flip[0] & 1]
                flip[0] += 1
                sra.sparse_lora_fwd(S, Xt, A, B, Y=Y, U=U, ws=ws)
            return one

        call_ms = time_graph(both, args.steps, args.warmup, not args.no_graph) / 2
        k_ms = time_kernel(SRA_KERNEL_DECODE24, alternate(main), max(20, args.steps))
        k2_ms = time_kernel(SRA_KERNEL_DECODE24, alternate(other), max(20, args.steps))
        # the same weight at 2:8 (its own decode kernel): streaming layout, and canonical arrays
        k28_ms = time_kernel(SRA_KERNEL_DECODE24, alternate(nm28t), max(20, args.steps))
        c28_ms = time_graph(lambda: [sra.sparse_lora_fwd(S, Xt, A, B, Y=Y, U=U, ws=ws) for S in nm28t],
                            args.steps, args.warmup, not args.no_graph) / 2
        k28c_ms = time_kernel(SRA_KERNEL_DECODE24, alternate(nm28), max(20, args.steps))
        kb28 = decode_bytes(wl, T, kernel_only=True, m=8)
        d_ms = time_graph(lambda: [torch.nn.functional.linear(Xt, Wd) for Wd in dense], args.steps,
                          args.warmup, not args.no_graph) / 2
        kb = decode_bytes(wl, T, kernel_only=True)
        rows.append({"T": T, "layout": args.decode_layout,
                     "call_us": round(call_ms * 1e3, 2), "kernel_us": round(k_ms * 1e3, 2),
                     "kernel_GBps": round(kb / (k_ms * 1e-3) / 1e9, 1),
                     "kernel_frac_hbm": round(kb / (k_ms * 1e-3) / PEAK_HBM_BPS, 4),
                     "call_GBps": round(decode_bytes(wl, T) / (call_ms * 1e-3) / 1e9, 1),
                     "dense_us": round(d_ms * 1e3, 2), "speedup_vs_dense": round(d_ms / call_ms, 3),
                     "other_layout_kernel_us": round(k2_ms * 1e3, 2),
                     "other_layout_frac_hbm": round(kb / (k2_ms * 1e-3) / PEAK_HBM_BPS, 4),
                     "nm28_kernel_us": round(k28_ms * 1e3, 2),
                     "nm28_kernel_GBps": round(kb28 / (k28_ms * 1e-3) / 1e9, 1),
                     "nm28_kernel_frac_hbm": round(kb28 / (k28_ms * 1e-3) / PEAK_HBM_BPS, 4),
                     "nm28_call_us": round(c28_ms * 1e3, 2),
                     "nm28_canonical_kernel_us": round(k28c_ms * 1e3, 2),
                     "nm28_traffic": TRAFFIC_BYTES.get(f"{wl.name}/T{T}/streaming/k_decode28<9,1>"),
                     "nm28_speedup_vs_dense": round(d_ms / c28_ms, 3)})
    return rows


def bench_update(args, wl):
    """Sparse update step on the OPT-66B FFN weight's compressed values (339.7 MB): the decayed SGD
    step Ws <- (1 - lr wd) Ws - lr dWs in place (sra_nm_axpby), HBM-bound: read Ws and dWs, write
    Ws.  Synthetic dWs of the same size; two weight copies alternate against the Infinity Cache."""
    import torch

    import sparse_rank_adapter_amd as sra
    from sparse_rank_adapter_amd._abi import SRA_KERNEL_NM_UPDATE

    dev = torch.device("cuda:0")
    n = wl.N * wl.K // 2
    g = torch.Generator(device=dev).manual_seed(0)
    ws = [torch.randn(n, device=dev, generator=g).to(torch.bfloat16) for _ in range(2)]
    dw = [torch.randn(n, device=dev, generator=g).to(torch.bfloat16) for _ in range(2)]
    flip = [0]

    def one():
        i = flip[0] & 1
        flip[0] += 1
        sra.nm_axpby(1.0 - 1e-4, ws[i], -1e-3, dw[i], out=ws[i])
    for _ in range(4):
        one()
    k_ms = time_kernel(SRA_KERNEL_NM_UPDATE, one, max(20, args.steps))
    nbytes = 3 * n * 2
    return {"workload": f"{wl.name} weight values ({n} bf16)", "kernel_ms": round(k_ms, 5),
            "GBps": round(nbytes / (k_ms * 1e-3) / 1e9, 1),
            "frac_hbm": round(nbytes / (k_ms * 1e-3) / PEAK_HBM_BPS, 4)}


def bench_ffi(args, wl):
    """Fixed fan-in layer: forward on the tiled ELL weight, backward dX on the tiled CSR transpose
    plus the adapter gradients.  Compression, the transpose and the tiling are setup, timed apart
    (once per mask).  The same calls on the untiled ELL / CSR forms, which tile into the workspace
    on every call, are timed beside them."""
    import torch

    import sparse_rank_adapter_amd as sra
    from sparse_rank_adapter_amd._abi import SRA_KERNEL_SPMM_FFI
    from sra_inputs import layer_inputs

    dev = torch.device("cuda:0")
    inp = layer_inputs(wl, seed=0)
    X, W, A, B, dY = (inp[k].to(dev) for k in ("X", "W", "A", "B", "dY"))
    T, r = wl.T, wl.r
    graph = not args.no_graph
    S = sra.compress_ffi(W, wl.ffi_k)
    ST = sra.ffi_transpose(S)
    St, STt = sra.ffi_tile(S), sra.ffi_tile(ST)
    ms_setup = time_graph(lambda: sra.compress_ffi(W, wl.ffi_k), max(5, args.steps // 5), 2, False)
    ms_tile = time_graph(lambda: (sra.ffi_tile(S), sra.ffi_tile(ST)), max(5, args.steps // 5), 2, False)
    Y = torch.empty((T, wl.N), dtype=X.dtype, device=dev)
    U = torch.empty((T, r), dtype=torch.float32, device=dev)
    grads = {"dX": torch.empty((T, wl.K), dtype=X.dtype, device=dev),
             "dA": torch.empty((r, wl.K), dtype=torch.float32, device=dev),
             "dB": torch.empty((wl.N, r), dtype=torch.float32, device=dev)}

    def calls(fw, bw):
        ws_f = torch.empty(max(1, sra.fwd_workspace(fw, T, r)), dtype=torch.uint8, device=dev)
        ws_b = torch.empty(max(1, sra.bwd_workspace(bw, T, r)), dtype=torch.uint8, device=dev)

        def fwd():
            sra.sparse_lora_fwd(fw, X, A, B, Y=Y, U=U, ws=ws_f)

        def bwd():
            sra.sparse_lora_bwd(bw, dY, X, U, A, B, ws=ws_b, out=grads)
        return fwd, bwd, ws_f.numel(), ws_b.numel()
    fwd, bwd, wsf_t, wsb_t = calls(St, STt)
    ms_fwd = time_graph(fwd, args.steps, args.warmup, graph)
    ms_bwd = time_graph(bwd, args.steps, args.warmup, graph)
    reps = max(10, args.steps)
    # the product kernel: each stage's A tile written from the entry lists, dense MFMA
    k_fwd = time_kernel(SRA_KERNEL_SPMM_FFI, fwd, reps)
    k_bwd = time_kernel(SRA_KERNEL_SPMM_FFI, bwd, reps)
    fwd_u, bwd_u, wsf_u, wsb_u = calls(S, ST)
    ms_fwd_u = time_graph(fwd_u, args.steps, args.warmup, graph)
    ms_bwd_u = time_graph(bwd_u, args.steps, args.warmup, graph)
    Wd = W.contiguous()
    d_fwd = time_graph(lambda: torch.nn.functional.linear(X, Wd), args.steps, args.warmup, graph)
    d_bwd = time_graph(lambda: torch.matmul(dY, Wd), args.steps, args.warmup, graph)
    sparse_flops = 2 * T * wl.N * wl.ffi_k
    dense_eq = 2 * (2 * T * wl.N * wl.K) + 2 * T * r * (wl.K + wl.N) + 4 * T * r * (wl.N + wl.K)
    return {"workload": wl.name, "T": T, "K": wl.K, "N": wl.N, "k": wl.ffi_k, "r": r,
            "format": "tiled (sra_ffi_tile)",
            "fwd_ms": round(ms_fwd, 5), "bwd_ms": round(ms_bwd, 5),
            "dense_eq_tflops": round(dense_eq / ((ms_fwd + ms_bwd) * 1e-3) / 1e12, 2),
            "spmm_fwd_kernel_ms": round(k_fwd, 5), "spmm_bwd_kernel_ms": round(k_bwd, 5),
            "spmm_fwd_stored_tflops": round(sparse_flops / (k_fwd * 1e-3) / 1e12, 2),
            # the product runs the dense flops of each stage's A tile on bf16 MFMA
            "spmm_fwd_frac_bf16_mfma": round(2 * T * wl.N * wl.K / (k_fwd * 1e-3) / PEAK_BF16_FLOPS, 4),
            "dense_fwd_ms": round(d_fwd, 5), "dense_dx_ms": round(d_bwd, 5),
            "speedup_vs_dense": round((d_fwd + d_bwd) / (ms_fwd + ms_bwd), 3),
            "workspace_bytes": {"fwd": wsf_t, "bwd": wsb_t, "fwd_untiled": wsf_u, "bwd_untiled": wsb_u},
            "untiled_fwd_ms": round(ms_fwd_u, 5), "untiled_bwd_ms": round(ms_bwd_u, 5),
            "speedup_vs_dense_untiled": round((d_fwd + d_bwd) / (ms_fwd_u + ms_bwd_u), 3),
            "compress_ffi_ms": round(ms_setup, 5), "ffi_tile_both_ms": round(ms_tile, 5)}


def bench_squash(args, wl):
    """SQuAsh's variant: the 2:4 layer with a rank-r adapter whose A keeps wl.adapter_k inputs per
    row (fixed fan-in, ELL values + int16 columns), against the same layer with a dense adapter of
    the same bytes (rank r_dense = adapter bytes / 2 (K + N)) and against the dense GEMMs."""
    import torch

    import sparse_rank_adapter_amd as sra
    from sra_inputs import layer_inputs

    dev = torch.device("cuda:0")
    inp = layer_inputs(wl, seed=0)
    X, W, Af, B, dY = (inp[k].to(dev) for k in ("X", "W", "A", "B", "dY"))
    T, r, k = wl.T, wl.r, wl.adapter_k
    graph = not args.no_graph
    S, P = sra.compress_pair(W)
    A = sra.compress_ffi(Af, k)
    ffa_bytes = r * k * (2 + 2) + wl.N * r * 2
    r_d = ffa_bytes // (2 * (wl.K + wl.N))
    Ad, Bd = Af[:r_d].contiguous(), B[:, :r_d].contiguous()
    Y = torch.empty((T, wl.N), dtype=X.dtype, device=dev)
    U = torch.empty((T, r), dtype=torch.float32, device=dev)
    Ud = torch.empty((T, r_d), dtype=torch.float32, device=dev)
    g = {"dX": torch.empty((T, wl.K), dtype=X.dtype, device=dev),
         "dA_values": torch.empty((r, k), dtype=torch.float32, device=dev),
         "dB": torch.empty((wl.N, r), dtype=torch.float32, device=dev)}
    gd = {"dX": torch.empty((T, wl.K), dtype=X.dtype, device=dev),
          "dA": torch.empty((r_d, wl.K), dtype=torch.float32, device=dev),
          "dB": torch.empty((wl.N, r_d), dtype=torch.float32, device=dev)}
    ws_f = torch.empty(max(1, sra.ffa_fwd_workspace(S, T, A), sra.fwd_workspace(S, T, r_d)),
                       dtype=torch.uint8, device=dev)
    ws_b = torch.empty(max(1, sra.ffa_bwd_workspace(P, T, A), sra.bwd_workspace(P, T, r_d)),
                       dtype=torch.uint8, device=dev)

    def fwd():
        sra.sparse_lora_fwd_ffa(S, X, A, B, Y=Y, U=U, ws=ws_f)

    def bwd():
        sra.sparse_lora_bwd_ffa(P, dY, X, U, A, B, ws=ws_b, out=g)

    def fwd_d():
        sra.sparse_lora_fwd(S, X, Ad, Bd, Y=Y, U=Ud, ws=ws_f)

    def bwd_d():
        sra.sparse_lora_bwd(P, dY, X, Ud, Ad, Bd, ws=ws_b, out=gd)
    fwd()
    bwd()
    fwd_d()
    bwd_d()
    ms_f = time_graph(fwd, args.steps, args.warmup, graph)
    ms_b = time_graph(bwd, args.steps, args.warmup, graph)
    ms_fd = time_graph(fwd_d, args.steps, args.warmup, graph)
    ms_bd = time_graph(bwd_d, args.steps, args.warmup, graph)
    Wd = W.contiguous()
    d_f = time_graph(lambda: torch.nn.functional.linear(X, Wd), args.steps, args.warmup, graph)
    d_b = time_graph(lambda: torch.matmul(dY, Wd), args.steps, args.warmup, graph)
    dense_eq = step_model(wl, T, with_compress=False)[0]
    return {"workload": wl.name, "T": T, "K": wl.K, "N": wl.N, "r": r, "adapter_k": k,
            "adapter_bytes": ffa_bytes, "dense_adapter_rank_same_bytes": r_d,
            "dense_adapter_bytes": r_d * 2 * (wl.K + wl.N),
            "fwd_ms": round(ms_f, 5), "bwd_ms": round(ms_b, 5),
            "dense_eq_tflops": round(dense_eq / ((ms_f + ms_b) * 1e-3) / 1e12, 2),
            "same_bytes_dense_adapter_fwd_ms": round(ms_fd, 5),
            "same_bytes_dense_adapter_bwd_ms": round(ms_bd, 5),
            "time_vs_same_bytes_dense_adapter": round((ms_f + ms_b) / (ms_fd + ms_bd), 3),
            "dense_fwd_gemm_ms": round(d_f, 5), "dense_dx_gemm_ms": round(d_b, 5),
            "speedup_vs_dense": round((d_f + d_b) / (ms_f + ms_b), 3)}


def loop_calls(args):
    """Repeat one call for counter collection: no timing, no output but a last line."""
    import torch

    import sparse_rank_adapter_amd as sra
    from sra_inputs import WORKLOADS, layer_inputs

    dev = torch.device("cuda:0")
    if args.loop == "read":
        # a plain reduction that reads 256 MiB (a ramp) and writes one value (counter calibration)
        a = torch.arange(64 << 20, dtype=torch.float32, device=dev)
        out = torch.empty((), dtype=torch.float32, device=dev)
        for _ in range(args.steps):
            torch.sum(a, dim=0, out=out)
        torch.cuda.synchronize()
        print(f"read 256 MiB x {args.steps}", flush=True)
        return
    if args.loop == "copy":
        # a plain elementwise kernel that reads 256 MiB (a ramp, no constant data) and writes 256 MiB
        a = torch.arange(64 << 20, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(args.steps):
            torch.neg(a, out=b)
        torch.cuda.synchronize()
        print(f"copy 256 MiB x {args.steps}", flush=True)
        return
    if args.loop == "mlp":
        # the chained OPT-13B MLP step's four products (streaming layout unless --layout canonical)
        w1, w2 = WORKLOADS["opt13b_fc1"], WORKLOADS["opt13b_fc2"]
        i1 = layer_inputs(w1, seed=0, with_dy=False)
        i2 = layer_inputs(w2, seed=0)
        X = i1["X"].to(dev)
        L = []
        for w, i in ((w1, i1), (w2, i2)):
            W, A, B = (i[k].to(dev) for k in ("W", "A", "B"))
            S, P = sra.compress_pair_tiled(W) if args.layout == "streaming" else sra.compress_pair(W)
            L.append((S, P, A, B))
        dY2 = i2["dY"].to(dev)
        for _ in range(args.steps):
            Y1, U1 = sra.sparse_lora_fwd(L[0][0], X, L[0][2], L[0][3])
            Y2, U2 = sra.sparse_lora_fwd(L[1][0], Y1, L[1][2], L[1][3])
            g2 = sra.sparse_lora_bwd(L[1][1], dY2, Y1, U2, L[1][2], L[1][3])
            sra.sparse_lora_bwd(L[0][1], g2["dX"], X, U1, L[0][2], L[0][3])
        torch.cuda.synchronize()
        print(f"mlp opt13b x {args.steps}", flush=True)
        return
    wl = WORKLOADS["opt66b_ffn_decode" if args.loop == "decode" else args.workload]
    T = args.decode_t if args.loop == "decode" else wl.T
    inp = layer_inputs(wl, seed=0, T=T, with_dy=args.loop == "spmm_bwd")
    X, W, A, B = (inp[k].to(dev) for k in ("X", "W", "A", "B"))
    n_, m_ = (int(x) for x in args.nm.split(":"))
    S = sra.compress(W, n_, m_)
    if args.loop == "decode" and args.decode_layout == "streaming":
        S = sra.nm_tile(S)
    Y, U = sra.sparse_lora_fwd(S, X, A, B)
    if args.loop == "spmm_bwd":
        P = sra.double_prune(S)
        dY = inp["dY"].to(dev)
        for _ in range(args.steps):
            sra.sparse_lora_bwd(P, dY, X, U, A, B)
    else:
        for _ in range(args.steps):
            sra.sparse_lora_fwd(S, X, A, B, Y=Y, U=U)
    torch.cuda.synchronize()
    print(f"{args.loop} {wl.name} T={T} x {args.steps}", flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library runs the layer on a single MI355X and has no "
              "multi-GPU path. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.workload == "opt13b_mlp" and args.nm != "2:4" and not args.loop:
        print("--nm applies to the single-layer workloads: the opt13b_mlp line is the 2:4 step and "
              "carries the same step on 2:8 weights as its nm28_opt13b_mlp extra", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.loop:
        loop_calls(args)
        return
    from sra_inputs import WORKLOADS
    if args.workload == "opt13b_mlp":
        out, (i1, i2) = bench_mlp_chain(args)
        extras(args, out, small=not args.no_small)
        m28, _ = bench_mlp_chain(args, inputs=(i1, i2), nm="2:8")
        out["nm28_opt13b_mlp"] = {k: m28[k] for k in (
            "value", "unit", "ms_per_step", "config", "speedup_vs_dense", "speedup_fwd_vs_dense_fwd",
            "speedup_bwd_vs_dense_dx", "detail_ms", "spmm_launches", "roofline", "engine_eval")
            if k in m28}
        if not args.no_cpu_baseline:
            out["cpu_baseline"] = cpu_baseline_mlp(i1, i2, args.cpu_budget)
            out["cpu_baseline_1thread"] = cpu_one_thread()
        print(json.dumps(out), flush=True)
        return
    wl = WORKLOADS[args.workload]
    if wl.name == "squash_opt350m_fc2":
        print(json.dumps(bench_squash(args, wl)), flush=True)
        return
    if wl.name == "ffi90_4096":
        print(json.dumps(bench_ffi(args, wl)), flush=True)
        return
    if wl.name == "opt66b_ffn_decode":
        rows = bench_decode(args, wl, (args.decode_t,))
        d = rows[0]
        out = {"metric": METRIC, "value": d["call_GBps"], "unit": "GB/s", "n_gpus": 1,
               "steps": args.steps, "warmup": args.warmup, "ms_per_step": d["call_us"] / 1e3,
               "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
               "data": "synthetic",
               "config": {"workload": wl.name, "T": args.decode_t, "K": wl.K, "N": wl.N, "r": wl.r,
                          "sparsity": "2:4", "layout": args.decode_layout,
                          "step": "forward (U = X A^T, Y = X Ws^T + U B^T)"},
               "decode": rows,
               "roofline": {"kernel": "k_decode24", "bound": "hbm", "achieved": d["kernel_GBps"],
                            "peak": PEAK_HBM_BPS / 1e9, "unit": "GB/s",
                            "frac": d["kernel_frac_hbm"],
                            "traffic": TRAFFIC_BYTES.get(
                                f"{wl.name}/T{args.decode_t}/{args.decode_layout}/k_decode24<3>")}}
        print(json.dumps(out), flush=True)
        return
    if wl.fmt != "nm":
        raise SystemExit(f"workload {wl.name} is not wired into bench.py yet")
    out, inp, dense_eq = bench_nm_layer(args, wl)
    extras(args, out, small=False)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, inp, args.cpu_budget, dense_eq)
        out["cpu_baseline"]["host"] = host_info()
    print(json.dumps(out), flush=True)


def extras(args, out, small):
    """The other workloads measured beside the headline line (each its own config)."""
    import copy

    from sra_inputs import WORKLOADS
    if small:
        sargs = copy.copy(args)
        sargs.layout = "canonical"
        s, _, _ = bench_nm_layer(sargs, WORKLOADS["opt350m_fc1"])
        keep = ("value", "unit", "ms_per_step", "config", "speedup_vs_dense",
                "speedup_step_incl_compress_vs_dense", "speedup_vs_dense_lora", "detail_ms",
                "speedup_fwd_vs_dense_fwd", "speedup_bwd_vs_dense_dx", "kernel_ms",
                "masked_weight_grad", "roofline", "replay_ms", "engine_eval", "added_zeros_frac")
        out["opt350m_fc1"] = {k: s[k] for k in keep if k in s}
        sargs.nm = "2:8"
        s8, _, _ = bench_nm_layer(sargs, WORKLOADS["opt350m_fc1"])
        out["nm28_opt350m_fc1"] = {k: s8[k] for k in keep if k in s8}
    if not args.no_decode:
        out["decode_opt66b_ffn"] = bench_decode(args, WORKLOADS["opt66b_ffn_decode"], (1, 4, 16))
        out["sparse_update_opt66b_ffn"] = bench_update(args, WORKLOADS["opt66b_ffn_decode"])
    if not args.no_ffi:
        out["ffi90_4096"] = bench_ffi(args, WORKLOADS["ffi90_4096"])
    out["squash_opt350m_fc2"] = bench_squash(args, WORKLOADS["squash_opt350m_fc2"])


if __name__ == "__main__":
    main()
