"""Shared helpers of the GPU tests: upload a workload, run pa_decode through the C ABI,
compare with the fp64 oracle."""
from __future__ import annotations

import os
import sys

import numpy as np

from decode_attention_paged_03_amd import pa
import oracle

# Accuracy bar for fp32 outputs: |gpu - oracle| <= 1e-3 * (1 + |oracle|) elementwise.
TOL = 1e-3


def oracle_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


class Device:
    """A workload's arrays on the GPU.  With ``guard`` a NaN page sits in front of each
    cache and the pointers handed to the library start one page in, so a stray -1 table
    entry would read NaN (and fail the comparison) instead of leaving the allocation.
    ``guard_after`` more NaN pages follow the pool (table entries just past the pool then
    also land on allocated NaN)."""

    def __init__(self, wl, guard: bool = True, guard_after: int = 0):
        import torch
        self.wl = wl
        dev = "cuda"
        page = wl.page_size * wl.kv_heads * wl.head_dim
        extra = 1 if guard else 0

        def cache(arr):
            t = torch.empty((wl.num_pages + extra + guard_after,) + arr.shape[1:],
                            dtype=torch.float16, device=dev)
            if guard:
                t[0].fill_(float("nan"))
            if guard_after:
                t[extra + wl.num_pages:].fill_(float("nan"))
            t[extra:extra + wl.num_pages].copy_(torch.from_numpy(arr))
            return t

        self.k_alloc = cache(wl.key_cache)
        self.v_alloc = cache(wl.value_cache)
        self.k = self.k_alloc[extra:extra + wl.num_pages]
        self.v = self.v_alloc[extra:extra + wl.num_pages]
        assert self.k.is_contiguous() and self.k.data_ptr() % 16 == 0 and page * 2 % 16 == 0
        self.q = torch.from_numpy(wl.query).to(dev)
        self.bt = torch.from_numpy(wl.block_tables).to(dev)
        self.ctx = torch.from_numpy(wl.context_lengths).to(dev)

    def run(self, dec, out=None):
        import torch
        if out is None:
            out = torch.full((self.wl.batch, self.wl.query_heads, self.wl.head_dim), float("nan"),
                             dtype=torch.float32, device="cuda")
        dec(self.q, self.k, self.v, self.bt, self.ctx, self.wl.scale, out=out)
        torch.cuda.synchronize()
        return out


def check_against_oracle(got: np.ndarray, ref: np.ndarray, what: str = ""):
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output at {np.argwhere(~np.isfinite(got))[:3]}"
    err = np.abs(got - ref)
    bound = TOL * (1.0 + np.abs(ref))
    worst = float((err / bound).max()) if err.size else 0.0
    say(f"[parity] {what}: max|err|={err.max() if err.size else 0:.3e} worst err/bound={worst:.3f}")
    assert worst <= 1.0, f"{what}: tolerance exceeded (err/bound {worst:.3f})"
    return worst


FIXED = pa.PA_FLAG_FIXED_PARTITIONS


def fixed_flags(partition_size) -> int:
    """The flag that keeps a partition size on the fixed-partition route (0 for none)."""
    return FIXED if partition_size else 0


def decode_and_check(wl, *, partition_size=None, flags=0, rows=None, guard=True, what=None):
    """pa_decode against the oracle.  A partition size given here means the fixed-partition
    route (PA_FLAG_FIXED_PARTITIONS); tests of the library's own choice pass the flag
    themselves through ``pa.decoder_for``."""
    what = what or wl.name
    if partition_size is None:
        partition_size = wl.partition_size
    if partition_size and not flags:
        flags = FIXED
    say(f"[case] {what}: {wl.summary()} partition={partition_size} flags={flags}")
    dev = Device(wl, guard=guard)
    dec = pa.decoder_for(wl, partition_size=partition_size, flags=flags)
    try:
        out = dev.run(dec).cpu().numpy()
    finally:
        dec.close()
    if rows is None:
        ref = oracle.attend_workload(wl, nthreads=oracle_threads())
        check_against_oracle(out, ref, what)
    else:
        ref = oracle.attend_workload(wl, rows=rows, nthreads=oracle_threads())
        check_against_oracle(out.reshape(-1, wl.head_dim)[rows], ref, what)
    return out
