"""Benchmark of the two-branch video sparse attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload full]
                    [--no-cpu-baseline] [--cpu-seconds 15]

One step = one whole vsa_forward (pool, [log-mass], coarse logits + softmax +
O_coarse, [tau], selection, fine attention + gated combine) on the full clip
shape: 32 heads, head_dim 128, prefix 512 text + 1536 reference-image + 256
reference-audio tokens, video grid 32x24x44 (33,792 tokens), keep 10%,
exact_kv_and_rows.  Inputs are seeded synthetic bf16 tensors, resident in HBM
before timing starts.  Prints one JSON line: the headline times plain forwards;
per-kernel times come from a second pass with HIP events between the kernels, and
ms_per_step_graph from replays of the same forward captured into a HIP graph.
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
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "fine_full_traffic.json"),
                    help="measured HBM bytes per fine launch (from rocprofv3 counters)")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the HIP-graph replay timing (ms_per_step_graph)")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="before timing, copy this many MiB device-to-device (a kernel of known "
                         "traffic that scales the FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


def cpu_baseline(w, x, target_s):
    """Time the fp64 oracle on a bounded sample of the same workload: heads in
    order, each with its pooling, coarse branch and selection and then the fine
    branch of its query tiles (dense and sparse alternately, in growing
    batches), until about target_s seconds have passed.  Reported as
    effective TFLOP/s over the sampled pairs."""
    from threadpoolctl import threadpool_info
    from oracle import vsa_oracle as O
    geom = O.map_geometry(w.segments(), *w.grid)
    sparse, dense = O.row_classes(geom, w.sink)
    order = []
    for i in range(max(len(sparse), len(dense))):
        if i < len(dense):
            order.append(dense[i])
        if i < len(sparse):
            order.append(sparse[i])
    dense_set = set(dense)
    k = O.keep_count(w.keep, geom.n_video)
    t0 = time.perf_counter()
    rows = 0
    pairs = 0
    heads = 0
    done = False
    for h in range(w.heads):
        Qh = O.bf16_bits_to_f64(x["q"][0, :, h])
        Kh = O.bf16_bits_to_f64(x["k"][0, :, h])
        Vh = O.bf16_bits_to_f64(x["v"][0, :, h])
        Gh = O.bf16_bits_to_f64(x["g"][0, :, h])
        heads += 1
        pos, n = 0, 1
        while pos < len(order):
            batch = order[pos:pos + n]
            O.forward_head(Qh, Kh, Vh, Gh, geom, w.keep, w.sink, w.select, w.coarse, w.tau, rows=batch)
            pos += len(batch)
            rows += len(batch)
            pairs += sum(geom.n_tiles if r in dense_set else geom.n_prefix + k for r in batch)
            if time.perf_counter() - t0 >= target_s:
                done = True
                break
            n = min(64, n * 2)
        if done:
            break
    el = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {
        "value": pairs * PAIR_FLOP / el / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"fp64 numpy oracle on the same inputs, heads taken in order ({heads} started): "
                   f"pooling + coarse + selection per head and the fine branch of {rows} query-tile rows "
                   f"({pairs} pairs of {w.heads * (geom.n_video * (geom.n_prefix + k) + geom.n_prefix * geom.n_tiles) if w.sink == 2 else 'n/a'}) "
                   f"in {el:.1f} s; dense and sparse rows alternate"),
        "seconds": round(el, 2),
    }


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {a.gpus})", file=sys.stderr)
        sys.exit(2)
    import torch
    import block_sparse_video_geometry_amd as V
    from workloads.synth import WORKLOADS, make_inputs

    w = WORKLOADS[a.workload]
    t0 = time.perf_counter()
    x = make_inputs(w)
    gen_s = time.perf_counter() - t0
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def to_dev(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v = to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"])
    g = to_dev(x["g"]) if x.get("g") is not None else None
    o = torch.empty_like(q)
    plan = V.vsa_plan_geometry(w.segments(), w.batch, *w.grid, w.heads, 128,
                               w.keep if w.keep > 0 else 100.0, sink=w.sink, select=w.select,
                               coarse=w.coarse, tau=w.tau, extra_tokens=w.extra)
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
                        f"{'exact_kv_and_rows' if w.sink == 2 else 'exact_kv'}",
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
        "kernels": kernels,
        "input_gen_s": round(gen_s, 1),
    }
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, x, a.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
