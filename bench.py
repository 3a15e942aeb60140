#!/usr/bin/env python3
"""Throughput of the fused forward pass of exact softmax attention on one MI355X.

One step = one call of the C-ABI entry point over the whole workload (every query row of
every (b, h)), with q/k/v already resident in device memory. Prints ONE JSON line.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--gpus 1] [--settle-s S]
                  [--entry fwd|splitkv [--num-splits S]] [--naive] [--backward] [--launch-loop C]

Before the W warm-up steps, untimed calls run for S seconds (default 0.2) so that the timed K
steps see the clock the chip sustains under load rather than its ramp-up.

The metric is forward TFLOP/s with 4*B*H*N^2*d flops per call (two products of
2*N^2*d per head, interactiveml.org "FlashAttention saves the matrix, not the quadratic
work"), halved for causal masks. Beside it: the roofline of the kernel (average kernel
duration from HIP events over the timed region, on the launch stream) and the fp64 CPU
oracle timed on a bounded sample of query rows on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from exact_softmax_attention_fa_amd import inputs  # noqa: E402

# MI355X published dense peaks (TFLOP/s): bf16 MFMA 2.5 PFLOP/s (256 CU x 2.4 GHz x 4096
# flop/clock), fp32 MFMA 157.3 TFLOP/s.
PEAK_TFLOPS = {"bf16": 2516.6, "f32": 157.3}
HBM_PEAK_GBS = 8000.0

CSRC = "exact_softmax_attention_fa_amd/csrc/"


def kernel_sources(w: inputs.Workload) -> list:
    """Sources of the kernel a workload runs (the key under which its traffic is stored): the
    kernel, the headers it includes and the front end that computes its launch arguments (for
    the tuned kernels also the bf16 dispatcher that routes widths 64 and 128 to them)."""
    if w.dtype == "f32":
        main = ["fa_fwd_f32.hip"]
    elif w.d == 128 or (w.d == 64 and w.B * w.H * -(-w.N // 256) >= 256):   # the tuned kernels
        main = ["fa_fwd_bf16_tuned.hip", "fa_dma.h", "fa_fwd_bf16.hip"]
    else:
        main = ["fa_fwd_bf16.hip"]
    return [CSRC + m for m in main + ["fa_internal.h", "fa_api.hip"]]


BACKWARD_SOURCES = [CSRC + m for m in ("fa_bwd_bf16.hip", "fa_bwd_internal.h", "fa_dma.h", "fa_api.hip")]


def sources_hash(rels: list) -> str:
    h = hashlib.sha256()
    for rel in rels:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# HBM bytes per launch measured with rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE (KiB per
# dispatch), each scaled by the factor the same counter reads for a plain copy of known size.
# Keyed by workload; valid only for the kernel sources whose hash is stored with them.
TRAFFIC = {
    "fwd_bf16_b1_h16_n8192_d128_widek": {"bytes": 202497544, "kernel_hash": "c367b38660587c73"},
}


def kernel_hash(w: inputs.Workload) -> str:
    return sources_hash(kernel_sources(w))


def library_info() -> dict:
    """The library file this process loads: its path, the sha256 of its bytes (first 16 hex
    digits) and whether it is the in-tree product build or a FA_LIBRARY override."""
    import exact_softmax_attention_fa_amd as fa
    path = fa.library_path()
    with open(path, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()[:16]
    override = "FA_LIBRARY" in os.environ
    info = {"sha16": sha, "product": not override}
    if override:
        info["path"] = path
    return info


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [p.get("num_threads", 0) for p in threadpool_info() if p.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:  # noqa: BLE001
        pass
    return os.cpu_count() or 1


def cpu_baseline(w: inputs.Workload, t: dict, rows_per_head: int) -> dict:
    """The fp64 oracle, as it stands, on `rows_per_head` evenly spaced query rows of every
    (b, h). Decoding the stored inputs to fp64 is done before the clock starts."""
    import numpy as np
    from oracle import attention as oracle
    q, k, v = (oracle.as_fp64(t[x], w.dtype) for x in "qkv")
    r = min(rows_per_head, w.N)
    rows = np.unique(np.linspace(0, w.N - 1, r).round().astype(np.int64))
    t0 = time.perf_counter()
    oracle.attention(q, k, v, w.resolved_scale(), w.causal, rows=rows)
    dt = time.perf_counter() - t0
    keys = (rows + 1) if w.causal else np.full(len(rows), w.N)
    flops = 4.0 * w.d * float(keys.sum()) * w.B * w.H
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": blas_threads(), "kind": "oracle",
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "sample": f"{len(rows)} of {w.N} query rows (evenly spaced) in each of {w.B * w.H} heads, "
                      f"fp64 numpy, {dt:.1f} s; flops counted per row as 4*d*visible keys"}


def copy_calibration(mib: int, steps: int) -> None:
    """A plain device-to-device copy of known size (reference for the HBM byte counters)."""
    import torch
    n = mib * (1 << 20) // 4
    x = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
    y = torch.empty_like(x)
    for _ in range(steps):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n * 4, "bytes_written": n * 4, "launches": steps}))


def naive_attention(q, kt, v, scale: float, causal: bool, mask=None):
    """Standard (unfused) attention as the pages describe it before FlashAttention: the N x N
    score matrix and the probability matrix are both written to and read back from HBM
    (sadullah.online, "Standard attention"; lihaoran.work, the intermediate matrix).
    Library GEMMs and a softmax kernel; a comparison only, never the product path.

    q, v: [B, H, N, d]; kt: K transposed to [B, H, d, N], contiguous (made once by the caller:
    a batched bf16 product with a transposed view as right operand is avoided). The scores are
    produced in fp32 (a bf16 x bf16 -> fp32 GEMM for bf16 inputs), as the fused kernel keeps
    them; the probabilities are rounded to the input dtype before the product with V, as the
    fused kernel rounds them."""
    import torch
    B, H, N, d = q.shape
    q3, kt3, v3 = q.reshape(B * H, N, d), kt.reshape(B * H, d, N), v.reshape(B * H, N, d)
    if q.dtype == torch.bfloat16:
        s = torch.bmm(q3, kt3, out_dtype=torch.float32)   # [B*H, N, N] fp32 in HBM
    else:
        s = torch.bmm(q3, kt3)
    s.mul_(scale)
    if causal:
        s.masked_fill_(mask, float("-inf"))
    p = torch.softmax(s, dim=-1).to(q.dtype)                  # [B*H, N, N] in HBM
    return torch.bmm(p, v3).reshape(B, H, N, d)


# Largest |naive - fused| the comparison is expected to show: both sides meet the oracle's
# bf16 bound (2e-2) or fp32 bound (1e-5), so they differ by at most twice that.
NAIVE_AGREEMENT = {"bf16": 4e-2, "f32": 2e-5}


def run_naive(w: inputs.Workload, q, k, v, o_fused, steps: int, warmup: int) -> dict:
    """Times the unfused comparison on the same device inputs (events over the timed region).
    The transposed copy of K is made once, before the timed region."""
    import torch
    mask = None
    if w.causal:
        mask = torch.ones(w.N, w.N, dtype=torch.bool, device=q.device).triu_(1)
    scale = w.resolved_scale()
    kt = k.transpose(-1, -2).contiguous()
    for _ in range(warmup):
        o = naive_attention(q, kt, v, scale, w.causal, mask)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(steps):
        o = naive_attention(q, kt, v, scale, w.causal, mask)
    ev1.record(stream)
    torch.cuda.synchronize()
    t = ev0.elapsed_time(ev1) / steps / 1e3
    diff = (o.float() - o_fused.float()).abs().max().item()
    return {"value": round(w.flops / t / 1e12, 2), "unit": "TFLOP/s", "ms_per_step": round(t * 1e3, 4),
            "kind": "naive: bmm (fp32 scores), softmax, bmm with the N x N matrices in HBM (torch)",
            "max_abs_diff_vs_fused": diff, "agrees_with_fused": diff <= NAIVE_AGREEMENT[w.dtype]}


def run_backward(w: inputs.Workload, q, k, v, o, lse, steps: int, warmup: int) -> dict:
    """Times fa_bwd (delta, dK/dV and dQ kernels) on the forward's own outputs; a seeded
    bf16 N(0,1) output gradient. Events on the launch stream over the timed region."""
    import numpy as np
    import torch
    import exact_softmax_attention_fa_amd as fa
    if w.dtype != "bf16" or w.d not in (64, 128):
        return {"skipped": "the backward pass supports bf16 with d = 64 or 128"}
    g = inputs.make_backward(w.B, w.H, w.N, w.d, w.seed + 100)["dout"]
    dout = torch.from_numpy(np.ascontiguousarray(g).view(np.int16)).view(torch.bfloat16).to(q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    delta = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=q.device)
    stream = torch.cuda.current_stream(q.device)
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(), lse.data_ptr(),
            dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(), w.B, w.H, w.N, w.d,
            w.resolved_scale(), 1 if w.causal else 0, stream.cuda_stream)

    def call():
        st = fa.fa_bwd(*args)
        if st != fa.FA_OK:
            raise fa.FaError(st, "fa_bwd")

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(steps):
        call()
    ev1.record(stream)
    torch.cuda.synchronize()
    t = ev0.elapsed_time(ev1) / steps / 1e3
    flops = 2.5 * w.flops   # five N^2 d products per head against the forward's two
    return {"value": round(flops / t / 1e12, 2), "unit": "TFLOP/s", "ms_per_step": round(t * 1e3, 4),
            "algorithmic_flops_per_call": flops, "sources_hash": sources_hash(BACKWARD_SOURCES),
            "note": "flops counted as 2.5x the forward (S recomputed once); the kernels compute S and dP "
                    "twice (dK/dV pass and dQ pass), 3.5x the forward's products",
            "pct_of_peak": round(100.0 * flops / t / 1e12 / PEAK_TFLOPS[w.dtype], 2)}


def run_launch_loop(entry, make_args, calls: int, o) -> dict:
    """Separates the launch cost from the kernel on short workloads (interactiveml.org,
    "FlashAttention saves the matrix, not the quadratic work": its closing list of measurements
    asks for kernel-launch, arithmetic and HBM time to be told apart). Three per-call
    times on the same inputs: one call at a time with a device synchronisation after each
    (host launch + kernel + completion), `calls` calls back to back (kernel + dispatch gap,
    HIP events on the launch stream), and the same launches replayed from a HIP graph of 100
    captured calls (no host launch path). The graph's output is checked bit for bit against
    the eager call's (the kernels are deterministic)."""
    import torch
    import exact_softmax_attention_fa_amd as fa

    def call(stream):
        st = entry(*make_args(stream.cuda_stream))
        if st != fa.FA_OK:
            raise fa.FaError(st, entry.__name__)

    stream = torch.cuda.current_stream()
    call(stream)
    torch.cuda.synchronize()
    eager = o.clone()
    n_sync = min(calls, 200)
    t0 = time.perf_counter()
    for _ in range(n_sync):
        call(stream)
        torch.cuda.synchronize()
    sync_us = (time.perf_counter() - t0) / n_sync * 1e6

    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(calls):
        call(stream)
    ev1.record(stream)
    torch.cuda.synchronize()
    loop_us = ev0.elapsed_time(ev1) / calls * 1e3

    per_graph = 100
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        cap = torch.cuda.current_stream()
        for _ in range(per_graph):
            call(cap)
    o.zero_()
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    matches = bool(torch.equal(o, eager))
    reps = max(1, calls // per_graph)
    ev0.record(stream)
    for _ in range(reps):
        graph.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    graph_us = ev0.elapsed_time(ev1) / (reps * per_graph) * 1e3
    matches = matches and bool(torch.equal(o, eager))
    return {"calls": calls, "sync_each_us": round(sync_us, 2), "back_to_back_us": round(loop_us, 2),
            "graph_replay_us": round(graph_us, 2), "graph_calls": reps * per_graph,
            "graph_output_matches_eager": matches}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=inputs.HEADLINE, choices=sorted(inputs.ALL_WORKLOADS))
    ap.add_argument("--settle-s", type=float, default=0.2,
                    help="untimed calls before the warm-up steps until the GPU has run this long "
                         "(the clock ramps up over the first tens of milliseconds)")
    ap.add_argument("--cpu-rows", type=int, default=8192,
                    help="query rows per head for the CPU oracle baseline (0 = skip)")
    ap.add_argument("--entry", default="fwd", choices=["fwd", "splitkv"],
                    help="entry point timed: the single-pass fa_fwd / fa_fwd_f32 (default) or "
                         "fa_fwd_splitkv (key range split over workgroups, then a merge)")
    ap.add_argument("--num-splits", type=int, default=0,
                    help="split columns requested from fa_fwd_splitkv (0 = the library's choice)")
    ap.add_argument("--backward", action="store_true",
                    help="also time the backward pass (fa_bwd) on the forward's outputs")
    ap.add_argument("--naive", action="store_true",
                    help="also time unfused standard attention on the same inputs (comparison)")
    ap.add_argument("--launch-loop", type=int, default=0, metavar="CALLS",
                    help="also separate launch cost from kernel time: CALLS calls synchronised one "
                         "by one, back to back, and replayed from a HIP graph")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain copy of MIB MiB --steps times (HBM counter reference)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(each GPU would run the same kernel on its own heads). Use --gpus 1.", file=sys.stderr)
        return 2

    if args.copy_calibration:
        copy_calibration(args.copy_calibration, args.steps)
        return 0

    import torch
    import exact_softmax_attention_fa_amd as fa

    w = inputs.ALL_WORKLOADS[args.workload]
    t = inputs.make(w)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def dev_tensor(x):
        import numpy as np
        if w.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(x).to(dev)

    q, k, v = (dev_tensor(t[x]) for x in "qkv")
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    split_info = None
    if args.entry == "splitkv":
        dtype_code = fa.FA_BF16 if w.dtype == "bf16" else fa.FA_F32
        st, nsplit, ws_bytes = fa.fa_fwd_splitkv_plan(w.B, w.H, w.N, w.d, dtype_code, 1 if w.causal else 0,
                                                      args.num_splits)
        if st != fa.FA_OK:
            raise fa.FaError(st, "fa_fwd_splitkv_plan")
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)   # allocated before timing
        split_info = {"requested": args.num_splits, "columns": nsplit, "workspace_bytes": ws_bytes}
        entry = fa.fa_fwd_splitkv

        def make_args(stream_handle):
            return (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                    w.B, w.H, w.N, w.d, w.resolved_scale(), 1 if w.causal else 0, dtype_code, args.num_splits,
                    ws.data_ptr(), ws_bytes, stream_handle)
    else:
        entry = fa.fa_fwd if w.dtype == "bf16" else fa.fa_fwd_f32

        def make_args(stream_handle):
            return (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                    w.B, w.H, w.N, w.d, w.resolved_scale(), 1 if w.causal else 0, stream_handle)
    call_args = make_args(stream.cuda_stream)

    def step():
        st = entry(*call_args)
        if st != fa.FA_OK:
            raise fa.FaError(st, entry.__name__)

    # The chip raises its clock over the first tens of milliseconds of sustained load (measured:
    # the headline kernel's first calls take up to 1.6x its steady time). Untimed calls run
    # until the GPU has been busy for --settle-s seconds, then the W warm-up steps, then the K
    # timed steps, so the timed region sees the sustained clock.
    settle_calls = 0
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < args.settle_s:
        for _ in range(4):
            step()
        settle_calls += 4
        torch.cuda.synchronize()
    settle_s = time.perf_counter() - t_settle
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # HIP events on the launch stream bracket the whole timed region (the launches run back to
    # back, so the region time / steps is the kernel's average duration plus the dispatch gap)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    avg_kernel_s = ev0.elapsed_time(ev1) / args.steps / 1e3
    ms_per_step = wall / args.steps * 1e3

    tflops = w.flops / (wall / args.steps) / 1e12
    achieved = w.flops / avg_kernel_s / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    kh = kernel_hash(w)
    lib = library_info()
    traffic = TRAFFIC.get(w.name)
    # stored counters hold only for the product build of the sources they were taken on
    traffic_bytes = (traffic["bytes"] if traffic and traffic.get("kernel_hash") == kh and lib["product"]
                     and args.entry == "fwd" else None)

    line = {
        "metric": "fwd attention TFLOP/s (4BHN^2d), bf16 N=8192 d=128; % of MFMA peak",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": w.causal,
                   "scale": w.resolved_scale(), "inputs": w.note, "seed": w.seed},
        "settle": {"seconds": round(settle_s, 3), "calls": settle_calls},
        "pct_of_peak": round(100.0 * tflops / peak, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4), "traffic": traffic_bytes,
                     "kernel_avg_us": round(avg_kernel_s * 1e6, 2),
                     "algorithmic_flops_per_launch": w.flops,
                     "algorithmic_bytes_per_launch": w.algorithmic_bytes,
                     "hbm_gbs_algorithmic": round(w.algorithmic_bytes / avg_kernel_s / 1e9, 1),
                     "kernel_hash": kh},
        "library": lib,
        "entry": entry.__name__,
        "cpu_baseline": None,
    }
    if split_info is not None:
        line["splitkv"] = split_info
        line["roofline"]["note"] = "kernel_avg_us covers both kernels of the call (partial pass and merge)"
    if not lib["product"]:
        line["non_product"] = "FA_LIBRARY override: not the in-tree build of the committed sources"
    if args.backward:
        line["backward"] = run_backward(w, q, k, v, o, lse, args.steps, args.warmup)
    if args.launch_loop > 0:
        line["launch"] = run_launch_loop(entry, make_args, args.launch_loop, o)
    if args.naive:
        nv = run_naive(w, q, k, v, o, args.steps, args.warmup)
        nv["fused_speedup"] = round(nv["ms_per_step"] / (avg_kernel_s * 1e3), 2)
        line["gpu_naive"] = nv
    if args.cpu_rows > 0:
        line["cpu_baseline"] = cpu_baseline(w, t, args.cpu_rows)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
