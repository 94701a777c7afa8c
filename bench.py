"""Benchmark of the two-branch video sparse attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload full]
                    [--no-cpu-baseline] [--cpu-workers 16] [--cpu-heads H] [--ceiling]

One step = one whole vsa_forward (pool, [log-mass], coarse logits + softmax +
O_coarse, [tau], selection, fine attention + gated combine) on the full clip
shape: 32 heads, head_dim 128, prefix 512 text + 1536 reference-image + 256
reference-audio tokens, video grid 32x24x44 (33,792 tokens), keep 10%,
exact_kv_and_rows.  Inputs are seeded synthetic bf16 tensors, resident in HBM
before timing starts.  Prints one JSON line: the headline times plain forwards;
per-kernel times come from a second pass with HIP events between the kernels, and
ms_per_step_graph from replays of the same forward captured into a HIP graph.
With --ceiling the line also carries, for context, what two library kernels reach on
the same device: a plain bf16 GEMM (torch.matmul, 8192^3) and torch's flash SDPA on
the dense shape of the workload (every token against every token, all heads).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PAIR_FLOP = 4 * 64 * 64 * 128          # QK^T + PV of one (query tile, key tile) pair
PEAK_BF16_TFLOPS = 2516.6               # MI355X dense bf16 MFMA (256 CU x 2.4 GHz x 4096 FLOP/clk)
PEAK_HBM_GBS = 8000.0
METRIC = "ms/layer and effective TFLOP/s (executed blocks) at 33.8k video tokens, 10% keep"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="full")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-workers", type=int, default=16,
                    help="most worker processes of the oracle's CPU baseline (one head per task)")
    ap.add_argument("--cpu-heads", type=int, default=None,
                    help="time the oracle on this many heads only (default: all, the whole forward)")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "fine_full_traffic.json"),
                    help="measured HBM bytes per fine launch (from rocprofv3 counters)")
    ap.add_argument("--no-dense", action="store_true",
                    help="skip timing the dense call (the dense-mode plan the schedule runs outside its window)")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the HIP-graph replay timing (ms_per_step_graph)")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="before timing, copy this many MiB device-to-device (a kernel of known "
                         "traffic that scales the FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--ceiling", action="store_true",
                    help="also time a plain bf16 GEMM and torch's flash SDPA on the workload's "
                         "dense shape (library kernels, for context)")
    return ap.parse_args()


def ceiling(torch, q, reps=3):
    """TFLOP/s of two library kernels on the current device, HIP events on the current
    stream: torch.matmul on 8192^3 bf16, and torch's flash SDPA (no other backend) with
    every query against every key of q's shape [batch, N, heads, 128] (random values)."""
    import torch.nn.functional as F
    from torch.nn.attention import SDPBackend, sdpa_kernel

    def timeit(fn, n):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    out = {}
    gen = torch.Generator(device=q.device).manual_seed(0)
    m = 8192
    x = torch.randn(m, m, device=q.device, dtype=torch.bfloat16, generator=gen)
    y = torch.randn(m, m, device=q.device, dtype=torch.bfloat16, generator=gen)
    gms = timeit(lambda: torch.matmul(x, y), 20)
    out["gemm_bf16_8192"] = {"ms": round(gms, 4), "tflops": round(2 * m ** 3 / (gms * 1e-3) / 1e12, 1)}
    del x, y
    B, N, H, D = q.shape
    qs = torch.randn(B, H, N, D, device=q.device, dtype=torch.bfloat16, generator=gen)
    ks, vs = torch.randn_like(qs), torch.randn_like(qs)
    try:
        with sdpa_kernel(SDPBackend.FLASH_ATTENTION):
            sms = timeit(lambda: F.scaled_dot_product_attention(qs, ks, vs), reps)
        out["sdpa_flash_dense"] = {"ms": round(sms, 3), "n_tokens": N, "heads": H,
                                   "tflops": round(4.0 * B * H * N * N * D / (sms * 1e-3) / 1e12, 1)}
    except RuntimeError as ex:
        out["sdpa_flash_dense"] = {"unavailable": str(ex)[:160]}
    return out


# inputs of the CPU baseline, read by forked workers (set before the pool starts)
_CPU_INPUTS = {}


def _oracle_head(h):
    """One (batch 0, head h) of the oracle's whole forward, single-threaded BLAS."""
    from threadpoolctl import threadpool_limits
    from oracle import vsa_oracle as O
    w, x = _CPU_INPUTS["w"], _CPU_INPUTS["x"]
    geom = O.map_geometry(w.segments(), *w.grid)
    t0 = time.perf_counter()
    with threadpool_limits(1):
        Qh, Kh, Vh = (O.bf16_bits_to_f64(x[n][0, :, h]) for n in "qkv")
        Gh = O.bf16_bits_to_f64(x["g"][0, :, h]) if x.get("g") is not None else None
        O.forward_head(Qh, Kh, Vh, Gh, geom, w.keep, w.sink, w.select, w.coarse, w.tau,
                       extra_tokens=w.extra)
    return time.perf_counter() - t0


def cpu_baseline(w, x, max_workers, heads=None):
    """Wall-clock of the fp64 oracle's whole forward on the same inputs (every head,
    every query tile: pooling, coarse branch, selection, fine branch and combine), one
    head per task over a pool of forked single-threaded workers on the host cores.
    Reported as effective TFLOP/s over the executed pairs, like the GPU figure.  Runs
    before anything touches the GPU, so the workers fork from a process without it."""
    import multiprocessing as mp
    from oracle import vsa_oracle as O
    geom = O.map_geometry(w.segments(), *w.grid)
    sparse, dense = O.row_classes(geom, w.sink)
    k = O.keep_count(w.keep, len(O.key_candidates(geom, w.sink)))
    n_heads = w.heads if heads is None else min(heads, w.heads)
    pairs = n_heads * (len(dense) * geom.n_tiles + len(sparse) * ((0 if w.sink == 0 else geom.n_prefix) + k))
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    workers = max(1, min(max_workers, avail, n_heads))
    _CPU_INPUTS.update(w=w, x=x)
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(workers) as pool:
        per_head = pool.map(_oracle_head, range(n_heads), chunksize=1)
    el = time.perf_counter() - t0
    _CPU_INPUTS.clear()
    return {
        "value": round(pairs * PAIR_FLOP / el / 1e12, 5),
        "unit": "TFLOP/s",
        "cores": workers,
        "kind": "oracle",
        "sample": (f"whole forward of the fp64 numpy oracle on the same inputs: {n_heads} of {w.heads} heads, "
                   f"every query tile ({pairs} executed pairs), one head per task on {workers} forked "
                   f"workers with single-threaded BLAS; wall-clock {el:.1f} s"),
        "seconds": round(el, 2),
        "ms_per_layer": round(1e3 * el, 1) if n_heads == w.heads else None,
        "head_seconds_mean": round(sum(per_head) / len(per_head), 2),
        "nproc": os.cpu_count(),
        "affinity_cores": avail,
    }


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {a.gpus})", file=sys.stderr)
        sys.exit(2)
    import torch
    from workloads.synth import WORKLOADS, make_inputs

    w = WORKLOADS[a.workload]
    t0 = time.perf_counter()
    x = make_inputs(w)
    gen_s = time.perf_counter() - t0
    # the CPU baseline first: its workers fork from a process that has not touched the GPU
    cpu = None
    if not a.no_cpu_baseline:
        print(f"[bench] cpu baseline: fp64 oracle, whole forward of {w.name}", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, x, a.cpu_workers, a.cpu_heads)
        print(f"[bench] cpu baseline done in {cpu['seconds']} s", file=sys.stderr, flush=True)
    import block_sparse_video_geometry_amd as V
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def to_dev(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v = to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"])
    g = to_dev(x["g"]) if x.get("g") is not None else None
    o = torch.empty_like(q)
    plan = V.vsa_plan_geometry(w.segments(), w.batch, *w.grid, w.heads, 128,
                               w.keep if w.keep > 0 else 100.0, sink=w.sink, select=w.select,
                               coarse=w.coarse, tau=w.tau, extra_tokens=w.extra, reblock=w.reblock)
    ws = V.alloc_workspace(plan)
    timer = V.Timer()
    stream = torch.cuda.current_stream()

    if a.calib_copy_mb > 0:
        n = a.calib_copy_mb << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(a.warmup):
        V.vsa_forward(plan, q, k, v, g, o, ws)
    torch.cuda.synchronize()
    stats = V.vsa_read_stats(plan, ws)
    def timed_steps(step):
        """Time exactly a.steps calls of step() with events on the launch stream."""
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(a.steps + 1)]
        torch.cuda.synchronize()
        evs[0].record(stream)
        for i in range(a.steps):
            step()
            evs[i + 1].record(stream)
        torch.cuda.synchronize()
        per_call = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(a.steps))
        med = per_call[len(per_call) // 2] if len(per_call) % 2 else 0.5 * (
            per_call[len(per_call) // 2 - 1] + per_call[len(per_call) // 2])
        return evs[0].elapsed_time(evs[-1]) / a.steps, med

    # the headline: plain forwards on the caller's stream
    ms, median_ms = timed_steps(lambda: V.vsa_forward(plan, q, k, v, g, o, ws))
    # per-kernel HIP-event times (the fine kernel's feeds the roofline line)
    timer.reset()
    timed_steps(lambda: V.vsa_forward_timed(plan, q, k, v, g, o, ws, timer))
    # the same forward captured once into a HIP graph and replayed
    graph_ms = None
    if not a.no_graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            V.vsa_forward(plan, q, k, v, g, o, ws)
        for _ in range(a.warmup):
            graph.replay()
        graph_ms, _ = timed_steps(graph.replay)
    kt = timer.read()
    # the dense call on the same inputs: every query tile over every key tile, no coarse branch
    dense = None
    if not a.no_dense:
        dplan = V.vsa_plan_geometry(w.segments(), w.batch, *w.grid, w.heads, 128, 100.0,
                                    select=V.VSA_SELECT_DENSE)
        dws = V.alloc_workspace(dplan)
        od = torch.empty_like(q)
        for _ in range(2):
            V.vsa_forward(dplan, q, k, v, None, od, dws)
        dstats = V.vsa_read_stats(dplan, dws)
        n_dense_calls = 5
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        evs[0].record(stream)
        for _ in range(n_dense_calls):
            V.vsa_forward(dplan, q, k, v, None, od, dws)
        evs[1].record(stream)
        torch.cuda.synchronize()
        dms = evs[0].elapsed_time(evs[1]) / n_dense_calls
        dense = {"ms_per_call": round(dms, 3), "calls": n_dense_calls,
                 "tflops": round(dstats["executed_pairs"] * PAIR_FLOP / (dms * 1e-3) / 1e12, 1),
                 "executed_pairs": dstats["executed_pairs"]}
        del od, dws, dplan
    flop = stats["executed_pairs"] * PAIR_FLOP
    tflops = flop / (ms * 1e-3) / 1e12

    fine_launches, fine_ms = kt["fine"]
    fine_avg_ms = fine_ms / fine_launches
    fine_tflops = flop / (fine_avg_ms * 1e-3) / 1e12
    # measured HBM bytes per fine launch, valid only for the kernel source the counters were
    # taken on (and the workload they were taken for)
    traffic = None
    if os.path.exists(a.traffic):
        with open(a.traffic) as f:
            t = json.load(f)
        src = os.path.join(ROOT, "block_sparse_video_geometry_amd", "csrc", "k_fine.hip")
        with open(src, "rb") as f:
            cur = hashlib.sha256(f.read()).hexdigest()[:16]
        if t.get("kernel_source_sha256_16") == cur and t.get("workload") == w.name:
            traffic = t.get("bytes_per_launch")
    kernels = {n: {"launches": c, "avg_us": 1e3 * t / max(c, 1)} for n, (c, t) in kt.items()}
    N, H = w.n_tokens, w.heads
    tensor_bytes = w.batch * N * H * 128 * 2
    pool_bytes = tensor_bytes * (1 + 2 * w.n_video / N)   # Q all tiles, K and V video tiles
    if "pool" in kernels:
        kernels["pool"]["gbs"] = pool_bytes / (kernels["pool"]["avg_us"] * 1e-6) / 1e9

    line = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms, 4),
        "ms_per_layer": round(ms, 4),
        "ms_per_layer_median": round(median_ms, 4),
        "ms_per_step_graph": round(graph_ms, 4) if graph_ms is not None else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded numpy normals rounded to bf16, shaped like the 1344x768 clips)",
        "config": {
            "workload": f"{w.name}: {H} heads x 128, prefix 512 text + 1536 ref-image + 256 ref-audio, "
                        f"video {w.grid[0]}x{w.grid[1]}x{w.grid[2]}, keep {w.keep:g}%, "
                        f"{'exact_kv_and_rows' if w.sink == 2 else 'exact_kv'}"
                        f"{', adaptive (reblocked) video tiles' if w.reblock else ''}",
            "batch": w.batch, "n_tokens": N, "video_tokens": w.n_video, "heads": H, "head_dim": 128,
            "executed_pairs": stats["executed_pairs"], "dense_pairs": stats["dense_pairs"],
            "k": stats["k"],
        },
        "roofline": {
            "kernel": "fine",
            "bound": "mfma",
            "achieved": round(fine_tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(fine_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "avg_launch_ms": round(fine_avg_ms, 4),
        },
        "whole_forward_frac_of_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "dense_call": dense,
        "sparse_speedup_vs_dense": round(dense["ms_per_call"] / ms, 2) if dense else None,
        "kernels": kernels,
        "input_gen_s": round(gen_s, 1),
    }
    if cpu is not None:
        line["cpu_baseline"] = cpu
    if a.ceiling:
        line["ceiling"] = ceiling(torch, q)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
