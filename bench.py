#!/usr/bin/env python3
"""Benchmark of one paged-attention decode step (pa_decode) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload batch64]

A step is one pa_decode call over the whole batch of the workload (all sequences, all
heads), with inputs resident in HBM.  To keep the 256 MB Infinity Cache from serving
the K/V reads, consecutive steps rotate over several identical copies of the K/V pools
(at least ~768 MB in total), so each step reads a copy that was evicted since its last
use.  The K timed steps are enqueued back to back; one pair of HIP events on the
library's stream brackets them, and the average call duration is that span / K.
Prints one JSON line.

HBM traffic (``roofline.traffic``) comes from rocprofv3 counter runs summarised under
profiles/ by ``python bench.py --summarize-pmc FETCH_DIR WRITE_DIR --workload W``; it is
reported only while the kernel sources still hash to what was profiled.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published peak
CSRC = os.path.join(ROOT, "decode_attention_paged_03_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")
COPY_BYTES = 256 * 1024 * 1024  # the calibration copy: reads and writes this many bytes
METRIC = "KV GB/s and % of HBM peak per decode step; decode tokens/s at batch 64"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="batch64",
                    choices=["tiny", "small_batch", "batch64", "long100k", "mixed128"])
    ap.add_argument("--partition", type=int, default=0,
                    help="partition_size: no partial covers more tokens (default 0: the library "
                         "splits the work; the library keeps its own split when that bound holds)")
    ap.add_argument("--fixed-partitions", action="store_true",
                    help="with --partition: partitions of exactly that size (PA_FLAG_FIXED_PARTITIONS)")
    ap.add_argument("--rotate-bytes", type=float, default=768e6,
                    help="total K/V bytes to rotate over (cold-cache timing); 0 = one copy")
    ap.add_argument("--append-steps", type=int, default=200,
                    help="calls of pa_append timed after the decode steps (0: skip)")
    ap.add_argument("--also", default="long100k,small_batch,mixed128,tiny",
                    help="comma-separated workloads measured after the headline one, each "
                         "reported in the line's \"workloads\" object ('none': only the headline)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=3.0,
                    help="target wall time of one oracle evaluation of the headline workload "
                         "(the other workloads use a third of it)")
    ap.add_argument("--write-resources", action="store_true",
                    help="compile the kernels with resource-usage remarks and write "
                         "profiles/resources.txt (no GPU needed)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy (for counter calibration)")
    ap.add_argument("--summarize-trace", metavar="TRACE_DIR",
                    help="turn a rocprofv3 --kernel-trace --stats output folder of this bench into "
                         "profiles/kernels_<workload>.txt")
    ap.add_argument("--summarize-counters", nargs="+", metavar="PMC_DIR",
                    help="turn rocprofv3 --pmc output folders of the COUNTER_PASSES into "
                         "profiles/counters_<workload>.txt")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two rocprofv3 --pmc output folders (FETCH_SIZE, WRITE_SIZE) of "
                         "`bench.py --copy-calibration` into profiles/traffic_<workload>.txt")
    return ap.parse_args()


def _code_only(text: str) -> str:
    """C++ source with comments removed and whitespace runs collapsed (string and character
    literals kept as they are), so that edits to comments leave the hash alone."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash() -> str:
    """sha256 over the code (comments and whitespace aside) of the decode kernels and their
    launch code: counters taken on other code do not apply.  (pa_append.hip holds a
    separate kernel, not part of a pa_decode call.)"""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".cpp", ".h")) and name != "pa_append.hip":
            with open(os.path.join(CSRC, name), encoding="utf-8") as f:
                h.update(name.encode() + b"\0" + _code_only(f.read()).encode())
    return h.hexdigest()


def _counter_rows(folder: str, counter: str):
    """Per-dispatch rows {Dispatch_Id, Kernel_Name, Counter_Value} of one counter from a
    rocprofv3 output folder (csv or the default SQLite database)."""
    rows = []
    for p in glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True):
        with open(p) as f:
            rows += [r for r in csv.DictReader(f) if r["Counter_Name"] == counter]
    if not rows:
        import sqlite3
        for p in glob.glob(os.path.join(folder, "**", "*.db"), recursive=True):
            db = sqlite3.connect(p)
            q = ("select dispatch_id, kernel_name, value from counters_collection "
                 "where counter_name = ?")
            rows += [{"Dispatch_Id": d, "Kernel_Name": k, "Counter_Value": v}
                     for d, k, v in db.execute(q, (counter,))]
            db.close()
    if not rows:
        raise SystemExit(f"no {counter} values under {folder}")
    return sorted(rows, key=lambda r: int(r["Dispatch_Id"]))


def summarize_pmc(fetch_dir: str, write_dir: str, workload: str) -> str:
    """KiB counters per dispatch -> bytes per pa_decode call.  The scale factor of each
    counter is what it reads for the plain copy of COPY_BYTES (the last dispatches of
    --copy-calibration) divided into COPY_BYTES."""
    out = {}
    for counter, folder in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _counter_rows(folder, counter)
        copies = [r for r in rows if "copyBuffer" in r["Kernel_Name"] or "copy" in r["Kernel_Name"].lower()]
        cal = float(copies[-1]["Counter_Value"]) * 1024.0
        factor = COPY_BYTES / cal
        pa_rows = [r for r in rows if re.search(r"\bpa_\w+", r["Kernel_Name"])]
        per_kernel = {}
        for r in pa_rows:
            m = re.search(r"(pa_\w+)", r["Kernel_Name"])
            name = m.group(1) if m else r["Kernel_Name"]
            per_kernel.setdefault(name, []).append(float(r["Counter_Value"]) * 1024.0 * factor)
        out[counter] = (factor, {k: sum(v) / len(v) for k, v in per_kernel.items()},
                        {k: len(v) for k, v in per_kernel.items()})
    # pa_append (timed after the decode steps) is not part of a pa_decode call
    fetch = sum(v for k, v in out["FETCH_SIZE"][1].items() if not k.startswith("pa_append"))
    write = sum(v for k, v in out["WRITE_SIZE"][1].items() if not k.startswith("pa_append"))
    lines = [f"# HBM traffic of one pa_decode call, workload {workload}",
             f"kernel_source_sha256: {kernel_source_hash()}",
             f"command_fetch: rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir> -o run -- python bench.py --workload {workload} "
             "--also none --steps 10 --warmup 2 --no-cpu-baseline --copy-calibration --append-steps 0",
             f"command_write: rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir> -o run -- python bench.py --workload {workload} "
             "--also none --steps 10 --warmup 2 --no-cpu-baseline --copy-calibration --append-steps 0",
             f"calibration: plain device copy of {COPY_BYTES} B; bytes = counter KiB * 1024 * factor",
             f"fetch_factor: {out['FETCH_SIZE'][0]:.4f}",
             f"write_factor: {out['WRITE_SIZE'][0]:.4f}"]
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        for k, v in out[counter][1].items():
            lines.append(f"{counter} {k}: {v:.0f} B per dispatch (mean of {out[counter][2][k]})")
    lines.append(f"fetch_bytes_per_call: {fetch:.0f}")
    lines.append(f"write_bytes_per_call: {write:.0f}")
    lines.append(f"traffic_bytes_per_call: {fetch + write:.0f}")
    path = os.path.join(PROFILES, f"traffic_{workload}.txt")
    os.makedirs(PROFILES, exist_ok=True)
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    return path


# Counter passes for LDS, occupancy and MFMA figures (each within one pass's hardware
# limits: at most 8 SQ and 2 GRBM counters).
COUNTER_PASSES = (("SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_INSTS_LDS", "SQ_WAVES",
                   "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "GRBM_GUI_ACTIVE"),
                  ("MeanOccupancyPerActiveCU", "MfmaUtil"),
                  ("TCC_EA0_RDREQ_sum", "TCC_EA0_RDREQ_32B_sum", "TCC_EA0_RDREQ_64B_sum",
                   "TCC_EA0_RDREQ_128B_sum"),
                  ("TCC_HIT_sum", "TCC_MISS_sum", "TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum",
                   "TCC_EA0_RDREQ_LEVEL_sum"),
                  ("SQ_WAVE_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY",
                   "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_VMEM", "SQ_ACTIVE_INST_LDS",
                   "SQ_ACTIVE_INST_SCA"),
                  ("SQ_INSTS_VALU", "SQ_INSTS_SALU", "SQ_INSTS_VMEM_RD", "SQ_INSTS_SMEM",
                   "SQ_WAIT_INST_LDS", "SQ_ACTIVE_INST_MISC", "SQ_WAVES"))


def summarize_counters(folders, workload: str) -> str:
    """Mean per dispatch of each counter of COUNTER_PASSES for the decode kernels, plus the
    LDS bank-conflict rate (conflict cycles over conflict-free active LDS cycles, as
    rocprofv3's LdsBankConflict), the share of HBM read requests that are whole 128-byte
    lines, and the mean read latency by Little's law (queue level over requests)."""
    names = [c for p in COUNTER_PASSES for c in p]
    per = {}
    for folder in folders:
        for c in names:
            try:
                rows = _counter_rows(folder, c)
            except SystemExit:
                continue
            for r in rows:
                m = re.search(r"(pa_\w+)(<[^(]*>)?", r["Kernel_Name"])
                if not m or m.group(1).startswith("pa_append"):
                    continue
                k = m.group(1) + (m.group(2) or "")
                per.setdefault(k, {}).setdefault(c, []).append(float(r["Counter_Value"]))
    if not per:
        raise SystemExit(f"no decode-kernel counter values under {folders}")
    lines = [f"# rocprofv3 counters of the decode kernels, workload {workload}",
             f"kernel_source_sha256: {kernel_source_hash()}"]
    for p in COUNTER_PASSES:
        lines.append(f"command: rocprofv3 --pmc {' '.join(p)} --output-format csv -d <dir> -o run -- "
                     f"python bench.py --workload {workload} --also none --steps 10 --warmup 2 "
                     "--no-cpu-baseline --append-steps 0")
    lines.append("(mean per dispatch, warm-up dispatches included)")
    for k, cs in per.items():
        lines.append(f"{k}:")
        for c in names:
            if c in cs:
                v = cs[c]
                lines.append(f"  {c}: {sum(v) / len(v):.6g} (mean of {len(v)})")
        bc = cs.get("SQ_LDS_BANK_CONFLICT")
        act = cs.get("SQ_LDS_IDX_ACTIVE")
        if bc and act and sum(act) > sum(bc):
            lines.append(f"  lds_bank_conflict_rate: {sum(bc) / (sum(act) - sum(bc)):.4f} "
                         "(conflict cycles per conflict-free active LDS cycle)")
        w = cs.get("SQ_WAVES")
        if w:
            lines.append(f"  waves_per_dispatch: {sum(w) / len(w):.0f}")
            for c in ("SQ_INSTS_VALU", "SQ_INSTS_SALU", "SQ_INSTS_VMEM_RD"):
                if c in cs:
                    lines.append(f"  {c.lower()}_per_wave: {sum(cs[c]) / len(cs[c]) / (sum(w) / len(w)):.0f}")
        rq, r128 = cs.get("TCC_EA0_RDREQ_sum"), cs.get("TCC_EA0_RDREQ_128B_sum")
        if rq and r128 and sum(rq) > 0:
            lines.append(f"  hbm_read_requests_128B_fraction: {sum(r128) / sum(rq):.4f}")
        lvl = cs.get("TCC_EA0_RDREQ_LEVEL_sum")
        if rq and lvl and sum(rq) > 0:
            lines.append(f"  mean_read_request_latency_l2_cycles: {sum(lvl) / sum(rq):.0f} "
                         "(accumulated queue level over requests)")
    path = os.path.join(PROFILES, f"counters_{workload}.txt")
    os.makedirs(PROFILES, exist_ok=True)
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    return path


def summarize_trace(folder: str, workload: str, steps: int = 200) -> str:
    """Per-kernel call count and average duration from rocprofv3's kernel statistics
    (stats csv, else the SQLite database's top_kernels view)."""
    stats = []
    for p in glob.glob(os.path.join(folder, "**", "*kernel_stats.csv"), recursive=True):
        with open(p) as f:
            for r in csv.DictReader(f):
                stats.append((r["Name"], int(r["Calls"]), float(r["AverageNs"]) / 1e3,
                              float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3))
    if not stats:
        import sqlite3
        for p in glob.glob(os.path.join(folder, "**", "*.db"), recursive=True):
            db = sqlite3.connect(p)
            q = ("select name, count(*), avg(end - start), min(end - start), max(end - start) "
                 "from kernels group by name order by sum(end - start) desc")
            stats += [(n, c, a / 1e3, lo / 1e3, hi / 1e3) for n, c, a, lo, hi in db.execute(q)]
            db.close()
    lines = [f"# rocprofv3 kernel statistics, workload {workload}",
             f"kernel_source_sha256: {kernel_source_hash()}",
             f"command: rocprofv3 --kernel-trace --stats --output-format csv -d <dir> -o run -- python bench.py "
             f"--workload {workload} --also none --steps {steps} --no-cpu-baseline",
             "(calls include the warm-up calls; durations in microseconds)",
             f"{'kernel':<48} {'calls':>6} {'avg_us':>9} {'min_us':>9} {'max_us':>9}"]
    per_call = 0.0
    for n, c, a, lo, hi in stats:
        m = re.search(r"(pa_\w+)(<[^(]*>)?", n)
        short = (m.group(1) + (m.group(2) or "")) if m else n[:48]
        lines.append(f"{short:<48} {c:>6} {a:>9.3f} {lo:>9.3f} {hi:>9.3f}")
        if m and not m.group(1).startswith("pa_append"):
            per_call += a
    lines.append(f"sum of the decode kernels' averages (one pa_decode call): {per_call:.3f} us")
    path = os.path.join(PROFILES, f"kernels_{workload}.txt")
    os.makedirs(PROFILES, exist_ok=True)
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    return path


def traffic_per_call(workload: str):
    """Bytes per call from profiles/traffic_<workload>.txt, or None when absent or taken
    on other kernel sources."""
    path = os.path.join(PROFILES, f"traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256") != kernel_source_hash():
        return None
    try:
        return float(kv["traffic_bytes_per_call"])
    except (KeyError, ValueError):
        return None


# The GPU machine gives one GPU a share of 16 host cores; the oracle never uses more threads.
CPU_SHARE = 16


def host_cores() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def cpu_baseline(wl, target_s: float, modes=("single", "all"), reps: int = 3):
    """Time the fp64 oracle (as it is) on the host cores over a bounded sample of the
    workload: output rows (sequence, query head) taken from the front of the batch until
    one evaluation should take about ``target_s``.  Each mode (one thread; all threads of
    the box's share) runs ``reps`` evaluations and reports the median.  A row's KV bytes
    count 1/group of its KV head's ctx * head_dim * 4 bytes, so whole sequences count what
    the GPU's KV-bytes metric counts."""
    import numpy as np
    import oracle
    threads_all = max(1, min(host_cores(), CPU_SHARE))
    ctx = wl.context_lengths.astype(np.int64)
    QH, G = wl.query_heads, wl.group
    # rows in b-major order, skipping empty sequences; probe one row of the first non-empty
    rows_all = [b * QH + h for b in range(wl.batch) if ctx[b] > 0 for h in range(QH)]
    if not rows_all:
        return None
    t0 = time.perf_counter()
    oracle.attend_workload(wl, rows=rows_all[:1], nthreads=1)
    per_token_row = (time.perf_counter() - t0) / max(1, int(ctx[rows_all[0] // QH]))
    out = {}
    for mode in modes:
        threads = 1 if mode == "single" else threads_all
        budget = target_s * threads / max(per_token_row, 1e-12)     # token-rows per evaluation
        rows, acc = [], 0
        for r in rows_all:
            c = int(ctx[r // QH])
            if rows and acc + c > budget:
                break
            rows.append(r)
            acc += c
        kv_bytes = acc * wl.head_dim * 4 / G
        times = []
        for _ in range(reps):
            t0 = time.perf_counter()
            oracle.attend_workload(wl, rows=rows, nthreads=threads)
            times.append(time.perf_counter() - t0)
        dt = float(np.median(times))
        nseq = len({r // QH for r in rows})
        out[mode] = {"value": round(kv_bytes / dt / 1e9, 6), "unit": "GB/s", "threads": threads,
                     "seconds_median": round(dt, 4), "evaluations": reps,
                     "sample": f"{len(rows)} of {len(rows_all)} output rows (first {nseq} "
                               f"sequences), {kv_bytes / 1e6:.2f} MB of K/V"}
    main_mode = "all" if "all" in out else "single"
    m = out[main_mode]
    line = {"value": m["value"], "unit": "GB/s", "cores": m["threads"], "host_cores": host_cores(),
            "kind": "oracle",
            "sample": f"{m['sample']}, median of {m['evaluations']} evaluation(s) on "
                      f"{m['threads']} OpenMP thread(s) (threads capped at the GPU box's "
                      f"{CPU_SHARE}-core share)"}
    line.update({k: v for k, v in out.items()})
    return line


def measure_append(dec, wl, k, v, bt, stream, steps: int):
    """Time pa_append, the step that stores each sequence's new key/value rows before the
    decode: every sequence rewrites the slot of its newest cached token with the bytes
    already there, so the caches (and later decodes) are unchanged.  Bytes per call: the
    new rows read and written (K and V), plus one position and one table entry per
    sequence."""
    import numpy as np
    import torch
    if steps <= 0:
        return None
    ps = wl.page_size
    last = wl.context_lengths.astype(np.int64) - 1
    live = last >= 0
    page = torch.from_numpy(np.where(live, wl.block_tables[np.arange(wl.batch),
                                                           np.maximum(last, 0) // ps], 0)
                            .astype(np.int64)).to(k.device)
    slot = torch.from_numpy(np.maximum(last, 0) % ps).to(k.device)
    new_k = k[page, slot].contiguous()
    new_v = v[page, slot].contiguous()
    pos = torch.from_numpy(np.where(live, last, -1).astype(np.int32)).to(k.device)
    for _ in range(5):
        dec.append(new_k, new_v, k, v, bt, pos, stream=stream)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    # eager: each call also pays the Python binding's enqueue cost, which is longer than
    # the kernel, so back-to-back calls measure the host
    start.record(stream)
    for _ in range(steps):
        dec.append(new_k, new_v, k, v, bt, pos, stream=stream)
    end.record(stream)
    torch.cuda.synchronize()
    us_eager = start.elapsed_time(end) / steps * 1e3
    # the same calls recorded once into a HIP graph and replayed: device time per call
    reps = 20
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(reps):
            dec.append(new_k, new_v, k, v, bt, pos)
    graph.replay()
    torch.cuda.synchronize()
    n_replay = max(1, steps // reps)
    cur = torch.cuda.current_stream()
    start.record(cur)
    for _ in range(n_replay):
        graph.replay()
    end.record(cur)
    torch.cuda.synchronize()
    us = start.elapsed_time(end) / (n_replay * reps) * 1e3
    n = int(live.sum())
    nbytes = 2 * 2 * n * wl.kv_heads * wl.head_dim * 2 + 2 * 4 * wl.batch
    return {"kernel": "pa_append_kernel", "us_per_call": round(us, 3),
            "us_per_call_eager": round(us_eager, 3),
            "bytes_per_call": nbytes, "GB/s": round(nbytes / (us * 1e-6) / 1e9, 3),
            "frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 6),
            "timing": f"HIP events around {n_replay} replays of a graph of {reps} calls "
                      f"(eager: {steps} back-to-back calls)"}


def resources_path() -> str:
    return os.path.join(PROFILES, "resources.txt")


def write_resources() -> str:
    """Compile the kernels with clang's resource-usage remarks (registers, scratch,
    occupancy, LDS per kernel) into profiles/resources.txt, keyed by the kernel sources'
    hash.  Needs no GPU."""
    import tempfile
    from decode_attention_paged_03_amd import build as B
    with tempfile.TemporaryDirectory() as d:
        B.build(asm_dir=d, out=os.path.join(d, "libpa.so"), build_dir=os.path.join(d, "_build"))
        with open(os.path.join(d, "resource_usage.txt")) as f:
            table = B.resource_table(f.read())
    lines = ["# Resource usage of the kernels (clang -Rpass-analysis=kernel-resource-usage, gfx950)",
             f"kernel_source_sha256: {kernel_source_hash()}",
             "command: python bench.py --write-resources",
             "(template arguments: decode kernels <head_dim, heads per wave, tile buffers, waves, "
             "pages of 8, whole-row K>; sgpr/vgpr/agpr per wave, scratch bytes per lane, "
             "waves/simd the registers allow, lds bytes per workgroup)",
             table]
    os.makedirs(PROFILES, exist_ok=True)
    with open(resources_path(), "w") as f:
        f.write("\n".join(lines) + "\n")
    return resources_path()


def kernel_resources(kernel_names):
    """Rows of profiles/resources.txt for the given kernels (e.g. 'pa_decode_balanced<128,4,1,12,0,1>'),
    or None when the file is absent or was written for other kernel sources."""
    path = resources_path()
    if not os.path.exists(path):
        return None
    with open(path) as f:
        text = f.read()
    m = re.search(r"kernel_source_sha256: (\w+)", text)
    if not m or m.group(1) != kernel_source_hash():
        return None
    lines = text.splitlines()
    hdr = next((l for l in lines if l.startswith("kernel ")), None)
    if hdr is None:
        return None
    cols = hdr.split()[1:]
    out = {}
    for l in lines:
        parts = l.split()
        if parts and parts[0] in kernel_names:
            out[parts[0]] = dict(zip(cols, (int(x) for x in parts[1:])))
    return out or None


def decode_kernel_names(wl, short: bool, cus: int = 256):
    """Names (as in profiles/resources.txt) of the kernels one pa_decode call runs on the
    library's own route: heads per wave = the largest divisor of the group up to 8; pages
    of 8 split a tile; whole-row K loads at head_dim 128 (when the LDS fits).  Short
    contexts (no workspace) take the fixed kernel with one partition per sequence -- 8
    waves when its grid (batch x KV heads x head chunks) fits the compute units, else 4 --
    and no merge."""
    hp = max(h for h in range(1, 9) if wl.group % h == 0)
    split = 1 if wl.page_size < 16 else 0
    if short:
        grid = wl.batch * wl.kv_heads * (wl.group // hp)
        return [f"pa_decode_kernel<{wl.head_dim},{hp},1,{8 if grid <= cus else 4},{split}>"]
    krow = 1 if wl.head_dim == 128 else 0
    return [f"pa_decode_balanced<{wl.head_dim},{hp},1,12,{split},{krow},0>",
            f"pa_merge_balanced<{wl.head_dim},{hp}>"]


def measure(W, pa, wl, args, stream, steps, warmup, append_steps=0, copy_calibration=False):
    """Time pa_decode on one workload: wall clock and HIP events around `steps`
    back-to-back calls over rotated cold copies of the K/V pools, plus single calls."""
    import numpy as np
    import torch
    fixed = bool(args.partition and args.fixed_partitions)
    dec = pa.decoder_for(wl, partition_size=args.partition,
                         flags=pa.PA_FLAG_FIXED_PARTITIONS if fixed else 0)
    dev = "cuda"
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

    # one bound call per pool copy: arguments checked and converted once, as a decode loop
    # would (the per-call Python checks would otherwise limit the smallest workloads)
    calls = [dec.bind(q, ks[j], vs[j], bt, ctx, wl.scale, out, stream=stream) for j in range(n_copies)]

    def step(i):
        calls[i % n_copies]()

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(steps):
        step(i)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    region_ms = start.elapsed_time(end)
    ms_per_step = wall / steps * 1e3
    value = kv_bytes / (ms_per_step * 1e-3) / 1e9
    avg_launch_ms = region_ms / steps
    achieved = kv_bytes / (avg_launch_ms * 1e-3) / 1e9

    # distribution of single calls: an event pair around each call, calls back to back
    n_single = min(steps, 200)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n_single)]
    for i, (e0, e1) in enumerate(evs):
        e0.record(stream)
        step(i)
        e1.record(stream)
    torch.cuda.synchronize()
    single_us = np.array([e0.elapsed_time(e1) * 1e3 for e0, e1 in evs])
    median_us = float(np.median(single_us))

    append_line = measure_append(dec, wl, ks[0], vs[0], bt, stream, append_steps)
    if copy_calibration:
        n = COPY_BYTES // 4
        src = torch.randn(n, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    balanced = dec.problem.partition_size == 0
    if balanced and dec.workspace_bytes == 0:
        kernel_name = "pa_decode call: pa_decode_kernel, one partition per sequence (short contexts, no merge)"
    elif balanced:
        kernel_name = "pa_decode call: pa_decode_balanced + pa_merge_balanced"
    elif fixed:
        kernel_name = "pa_decode call: pa_decode_kernel (+ pa_merge_kernel when split)"
    else:
        kernel_name = (f"pa_decode call with partition_size {args.partition}: the balanced kernels "
                       "when their partials fit it, else pa_decode_kernel + pa_merge_kernel")
    traffic = traffic_per_call(wl.name) if args.partition == 0 else None
    res = {
        "value": round(value, 3),
        "unit": "GB/s",
        "ms_per_step": round(ms_per_step, 6),
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 3),
        "tokens_per_s": round(wl.batch / (ms_per_step * 1e-3), 1),
        "config": {
            "workload": wl.name,
            "batch": wl.batch, "query_heads": wl.query_heads, "kv_heads": wl.kv_heads,
            "head_dim": wl.head_dim, "page_size": wl.page_size,
            "context_lengths": {"min": int(wl.context_lengths.min()),
                                "max": int(wl.context_lengths.max()),
                                "sum": int(wl.context_lengths.astype(np.int64).sum())},
            "partition_size": dec.problem.partition_size or "library default",
            "fixed_partitions": fixed,
            "kv_dtype": "f16", "out_dtype": "f32",
            "kv_bytes_per_step": kv_bytes,
            "kv_pool_copies_rotated": n_copies,
            "seed": wl.seed,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 3),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 5),
            "traffic": traffic,
            "kernel": kernel_name,
            "avg_launch_us": round(avg_launch_ms * 1e3, 3),
            "call_us_p10_median_p90": [round(float(np.percentile(single_us, q)), 3) for q in (10, 50, 90)],
            "frac_single_call_median": round(kv_bytes / (median_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 5),
            "timing": f"HIP events on the call's stream around {steps} back-to-back calls",
        },
    }
    if balanced:
        # the default route needs no workspace only when it takes one partition per sequence
        cus = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
        res["roofline"]["resources"] = kernel_resources(decode_kernel_names(wl, dec.workspace_bytes == 0, cus))
    if append_line:
        res["append"] = append_line
    dec.close()
    del ks, vs, k0, v0, q, bt, ctx, out
    torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace, args.workload))
        return
    if args.summarize_pmc:
        print(summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.workload))
        return
    if args.summarize_counters:
        print(summarize_counters(args.summarize_counters, args.workload))
        return
    if args.write_resources:
        print(write_resources())
        return
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only (asked for --gpus {args.gpus}); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch

    from decode_attention_paged_03_amd import pa
    from decode_attention_paged_03_amd import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    pa.load()
    stream = torch.cuda.current_stream()

    also = [] if args.also in ("", "none") else \
        [w for w in args.also.split(",") if w and w != args.workload]
    for w in also:
        if w not in W.WORKLOADS:
            raise SystemExit(f"bench.py: unknown workload {w!r} in --also")

    wl = W.make_named(args.workload)
    head = measure(W, pa, wl, args, stream, args.steps, args.warmup, args.append_steps,
                   args.copy_calibration)
    line = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": head["config"],
        "pct_hbm_peak": head["pct_hbm_peak"],
        "tokens_per_s": head["tokens_per_s"],
        "roofline": head["roofline"],
    }
    if "append" in head:
        line["append"] = head["append"]
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    del wl
    # the other workloads: same protocol, fewer steps, each in the "workloads" object
    others = {}
    for name in also:
        wl = W.make_named(name)
        r = measure(W, pa, wl, args, stream, min(args.steps, 200), args.warmup)
        if not args.no_cpu_baseline:
            big = name == "mixed128"
            r["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds / 3.0,
                                             modes=("all",) if big else ("single", "all"),
                                             reps=1 if big else 3)
        others[name] = r
        del wl
    if others:
        line["workloads"] = others
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
