#!/usr/bin/env python3
"""Benchmark of one paged-attention decode step (pa_decode) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload batch64]

A step is one pa_decode call over the whole batch of the workload (all sequences, all
heads), with inputs resident in HBM.  To keep the 256 MB Infinity Cache from serving
the K/V reads, consecutive steps rotate over several identical copies of the K/V pools
(at least ~768 MB in total), so each step reads a copy that was evicted since its last
use.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published peak
METRIC = "KV GB/s and % of HBM peak per decode step; decode tokens/s at batch 64"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="batch64",
                    choices=["tiny", "small_batch", "batch64", "long100k", "mixed128"])
    ap.add_argument("--partition", type=int, default=None,
                    help="tokens per partition (default: the workload's, else the library's)")
    ap.add_argument("--rotate-bytes", type=float, default=768e6,
                    help="total K/V bytes to rotate over (cold-cache timing); 0 = one copy")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy (for counter calibration)")
    return ap.parse_args()


def cpu_baseline(wl, target_s: float):
    """Time the fp64 oracle (as it is) on the host cores over a bounded sample of the
    workload: whole sequences (all query heads) from the front of the batch."""
    import numpy as np
    import oracle
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    cores = max(1, min(cores, 16))
    QH = wl.query_heads
    # probe on the first sequence to size the sample
    t0 = time.perf_counter()
    oracle.attend_workload(wl, rows=list(range(QH)), nthreads=cores)
    probe = time.perf_counter() - t0
    per_token = probe / max(1, int(wl.context_lengths[0]))
    budget_tokens = target_s / max(per_token, 1e-12)
    n, acc = 0, 0
    while n < wl.batch and acc + int(wl.context_lengths[n]) <= budget_tokens:
        acc += int(wl.context_lengths[n])
        n += 1
    n = max(n, 1)
    rows = list(range(n * QH))
    t0 = time.perf_counter()
    oracle.attend_workload(wl, rows=rows, nthreads=cores)
    dt = time.perf_counter() - t0
    kv_bytes = int(np.asarray(wl.context_lengths[:n], dtype=np.int64).sum()) * wl.kv_heads * wl.head_dim * 4
    return {"value": round(kv_bytes / dt / 1e9, 6), "unit": "GB/s", "cores": cores,
            "kind": "oracle",
            "sample": f"first {n} of {wl.batch} sequences (all {QH} query heads, "
                      f"{kv_bytes / 1e6:.1f} MB of K/V), {dt:.1f} s wall"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only (asked for --gpus {args.gpus}); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from decode_attention_paged_03_amd import pa
    from decode_attention_paged_03_amd import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    pa.load()

    wl = W.make_named(args.workload)
    part = args.partition if args.partition is not None else None
    dec = pa.decoder_for(wl, partition_size=part)
    dev = "cuda"
    stream = torch.cuda.current_stream()

    q = torch.from_numpy(wl.query).to(dev)
    bt = torch.from_numpy(wl.block_tables).to(dev)
    ctx = torch.from_numpy(wl.context_lengths).to(dev)
    k0 = torch.from_numpy(wl.key_cache).to(dev)
    v0 = torch.from_numpy(wl.value_cache).to(dev)
    kv_bytes = wl.kv_bytes()
    pool_bytes = 2 * k0.numel() * 2
    n_copies = 1 if args.rotate_bytes <= 0 else max(1, min(16, math.ceil(args.rotate_bytes / pool_bytes)))
    ks, vs = [k0], [v0]
    for _ in range(n_copies - 1):
        ks.append(k0.clone())
        vs.append(v0.clone())
    out = torch.empty((wl.batch, wl.query_heads, wl.head_dim), dtype=torch.float32, device=dev)

    def step(i):
        j = i % n_copies
        dec(q, ks[j], vs[j], bt, ctx, wl.scale, out=out, stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step(i)
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_ms = np.array([s.elapsed_time(e) for s, e in zip(starts, ends)])

    ms_per_step = wall / args.steps * 1e3
    value = kv_bytes / (ms_per_step * 1e-3) / 1e9
    avg_launch_ms = float(launch_ms.mean())
    achieved = kv_bytes / (avg_launch_ms * 1e-3) / 1e9

    if args.copy_calibration:
        n = 64 * 1024 * 1024
        src = torch.randn(n, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": wl.name,
            "batch": wl.batch, "query_heads": wl.query_heads, "kv_heads": wl.kv_heads,
            "head_dim": wl.head_dim, "page_size": wl.page_size,
            "context_lengths": {"min": int(wl.context_lengths.min()),
                                "max": int(wl.context_lengths.max()),
                                "sum": int(wl.context_lengths.astype(np.int64).sum())},
            "partition_size": dec.problem.partition_size or "library default",
            "kv_dtype": "f16", "out_dtype": "f32",
            "kv_bytes_per_step": kv_bytes,
            "kv_pool_copies_rotated": n_copies,
            "seed": wl.seed,
        },
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 3),
        "tokens_per_s": round(wl.batch / (ms_per_step * 1e-3), 1),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 3),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 5),
            "traffic": None,
            "kernel": "pa_decode (all kernels of one call)",
            "avg_launch_us": round(avg_launch_ms * 1e3, 3),
            "p10_us": round(float(np.percentile(launch_ms, 10)) * 1e3, 3),
            "p90_us": round(float(np.percentile(launch_ms, 90)) * 1e3, 3),
        },
    }
    dec.close()
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
