"""Seeded synthetic inputs for paged decode attention.

This module only *draws* inputs: context lengths, a physical-page assignment,
fp16 query / key / value values and canary fills.  It holds none of the
attention arithmetic, so both the HIP path and the CPU oracle can be fed from
it without sharing any of the method.

Layout (the "Data Layout" section of the "[TIL] Optimizing paged attention"
page): the K and V caches are pools of physical pages, each page holding
``page_size`` consecutive tokens, each token holding ``kv_heads`` vectors of
``head_dim`` fp16 values, i.e. ``[num_pages][page_size][kv_heads][head_dim]``.
A per-sequence block table (``[batch][max_pages_per_sequence]`` int32) maps a
logical page to a physical one; token ``t`` of a sequence lives in logical page
``t // page_size``, slot ``t % page_size``.  Unused table slots hold -1.

Draw order for every workload (one ``numpy.random.Generator(PCG64(seed))``):
context lengths -> page permutation -> query -> key -> value -> outlier rows.
Values are drawn in float32 and rounded to fp16 (round-to-nearest-even); the
fp16 bit patterns are what both sides consume.

Canaries (``canary=True``): every pool page that no sequence references and
every slot past the last valid token of a sequence's last page is filled with
an fp16 quiet NaN (0x7E00) in both K and V, so any read of memory outside the
valid token set poisons the output.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np

FP16_QNAN = np.uint16(0x7E00)


@dataclasses.dataclass
class Workload:
    name: str
    batch: int
    query_heads: int
    kv_heads: int
    head_dim: int
    page_size: int
    max_pages_per_sequence: int
    num_pages: int
    query: np.ndarray            # float16 [batch][query_heads][head_dim]
    key_cache: np.ndarray        # float16 [num_pages][page_size][kv_heads][head_dim]
    value_cache: np.ndarray      # float16 same layout as key_cache
    block_tables: np.ndarray     # int32 [batch][max_pages_per_sequence], -1 = unused
    context_lengths: np.ndarray  # int32 [batch]
    scale: float                 # exactly representable in float32
    partition_size: int = 0      # 0 = let the engine choose
    seed: int = 0

    @property
    def group(self) -> int:
        return self.query_heads // self.kv_heads

    @property
    def max_context_length(self) -> int:
        return int(self.context_lengths.max()) if self.batch else 0

    def kv_bytes(self) -> int:
        """K+V bytes the valid tokens occupy: sum(ctx) * kv_heads * head_dim * 2 (K,V) * 2 B."""
        return int(self.context_lengths.astype(np.int64).sum()) * self.kv_heads * self.head_dim * 4

    def summary(self) -> dict:
        return dict(name=self.name, batch=self.batch, query_heads=self.query_heads,
                    kv_heads=self.kv_heads, head_dim=self.head_dim, page_size=self.page_size,
                    max_pages_per_sequence=self.max_pages_per_sequence, num_pages=self.num_pages,
                    partition_size=self.partition_size, seed=self.seed,
                    ctx_min=int(self.context_lengths.min()) if self.batch else 0,
                    ctx_max=self.max_context_length,
                    ctx_sum=int(self.context_lengths.astype(np.int64).sum()))


def _fp16_fill(rng: np.random.Generator, shape, dist: str, chunk: int = 1 << 24,
               factor: float = 1.0) -> np.ndarray:
    """Draw ``prod(shape)`` values in float32, multiply them by ``factor`` and round to fp16
    once, in sequential chunks (a Generator draws the same stream whether asked for it at
    once or in pieces)."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float16)
    pos = 0
    while pos < n:
        m = min(chunk, n - pos)
        if dist == "normal":
            x = rng.standard_normal(m, dtype=np.float32)
        elif dist == "uniform":
            x = rng.random(m, dtype=np.float32) * np.float32(2.0) - np.float32(1.0)
        elif dist == "t3":
            # heavy tails: Student's t with 3 degrees of freedom
            x = rng.standard_t(3.0, m).astype(np.float32)
        else:
            raise ValueError(f"unknown distribution {dist!r}")
        if factor != 1.0:
            x = x * np.float32(factor)
        if dist == "t3" or factor != 1.0:
            x = np.clip(x, np.float32(-6e4), np.float32(6e4))   # inside fp16's finite range
        out[pos:pos + m] = x
        pos += m
    return out.reshape(shape)


def make_workload(*, name: str, batch: int, query_heads: int, kv_heads: int, head_dim: int,
                  page_size: int, context_lengths: Optional[Sequence[int]] = None,
                  ctx_sampler=None, max_pages_per_sequence: Optional[int] = None,
                  pool: str = "exact", pool_pages: Optional[int] = None, dist: str = "normal",
                  scale: Optional[float] = None, seed: int = 0, canary: bool = True,
                  outlier_fraction: float = 0.0, outlier_factor: float = 8.0,
                  partition_size: int = 0, v_dist: Optional[str] = None, v_factor: float = 1.0,
                  k_factor: float = 1.0) -> Workload:
    """Build one seeded paged-decode workload.

    ``context_lengths`` fixes the lengths; otherwise ``ctx_sampler(rng, batch)`` draws them.
    ``pool``: "exact" -> pool = pages needed; "holes10" -> ceil(1.1 * pages needed);
    an explicit ``pool_pages`` overrides both.  Pages are a seeded permutation of the pool,
    handed out in logical order (sequence 0's pages first), the rest are holes.
    ``outlier_fraction``: that fraction (rounded) of each sequence's token positions, chosen
    without replacement, has its K rows multiplied by ``outlier_factor`` for every KV head
    (a power of two keeps the product exact in fp16).
    ``v_dist`` / ``v_factor``: the value rows' distribution ("normal", "uniform" or "t3";
    default ``dist``) and a factor applied before rounding (wide value rows);
    ``k_factor``: a factor on the key rows before rounding (a small one gives near-tied
    scores).  At their defaults the draws are those of ``dist`` alone.
    """
    if query_heads % kv_heads:
        raise ValueError("query_heads must be a multiple of kv_heads")
    rng = np.random.Generator(np.random.PCG64(seed))
    if context_lengths is not None:
        ctx = np.asarray(context_lengths, dtype=np.int64).reshape(batch)
    else:
        ctx = np.asarray(ctx_sampler(rng, batch), dtype=np.int64).reshape(batch)
    if (ctx < 0).any():
        raise ValueError("negative context length")
    pages_per_seq = (ctx + page_size - 1) // page_size
    if max_pages_per_sequence is None:
        max_pages_per_sequence = max(1, int(pages_per_seq.max()) if batch else 1)
    if batch and pages_per_seq.max() > max_pages_per_sequence:
        raise ValueError("context longer than max_pages_per_sequence * page_size")
    needed = int(pages_per_seq.sum())
    if pool_pages is not None:
        num_pages = int(pool_pages)
    elif pool == "exact":
        num_pages = needed
    elif pool == "holes10":
        num_pages = (11 * needed + 9) // 10      # ceil(1.1 * needed) in integers
    else:
        raise ValueError(f"unknown pool rule {pool!r}")
    num_pages = max(num_pages, 1)
    if num_pages < needed:
        raise ValueError("pool smaller than the pages the sequences need")

    perm = rng.permutation(num_pages).astype(np.int64)
    bt = np.full((batch, max_pages_per_sequence), -1, dtype=np.int32)
    cursor = 0
    for b in range(batch):
        n = int(pages_per_seq[b])
        bt[b, :n] = perm[cursor:cursor + n]
        cursor += n

    q = _fp16_fill(rng, (batch, query_heads, head_dim), dist)
    kv_shape = (num_pages, page_size, kv_heads, head_dim)
    k = _fp16_fill(rng, kv_shape, dist, factor=k_factor)
    v = _fp16_fill(rng, kv_shape, dist if v_dist is None else v_dist, factor=v_factor)

    if outlier_fraction > 0.0:
        for b in range(batch):
            L = int(ctx[b])
            n_out = int(round(outlier_fraction * L))
            if n_out == 0:
                continue
            toks = rng.choice(L, size=n_out, replace=False)
            phys = bt[b, toks // page_size].astype(np.int64)
            slot = toks % page_size
            k[phys, slot] = k[phys, slot] * np.float16(outlier_factor)

    if canary:
        used = np.zeros(num_pages, dtype=bool)
        used[perm[:needed]] = True
        kb = k.view(np.uint16)
        vb = v.view(np.uint16)
        kb[~used] = FP16_QNAN
        vb[~used] = FP16_QNAN
        for b in range(batch):
            L = int(ctx[b])
            n = int(pages_per_seq[b])
            if n == 0:
                continue
            tail = L - (n - 1) * page_size
            if tail < page_size:
                last = int(bt[b, n - 1])
                kb[last, tail:] = FP16_QNAN
                vb[last, tail:] = FP16_QNAN

    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    scale = float(np.float32(scale))
    return Workload(name=name, batch=batch, query_heads=query_heads, kv_heads=kv_heads,
                    head_dim=head_dim, page_size=page_size,
                    max_pages_per_sequence=max_pages_per_sequence, num_pages=num_pages,
                    query=q, key_cache=k, value_cache=v, block_tables=bt,
                    context_lengths=ctx.astype(np.int32), scale=scale,
                    partition_size=partition_size, seed=seed)


# --------------------------------------------------------------------------------------
# The five reference workloads.  Seeds are 1000 + workload number.
# --------------------------------------------------------------------------------------

def _uniform_int(lo: int, hi: int):
    return lambda rng, n: rng.integers(lo, hi + 1, size=n)


def _lognormal_clipped(mu: float, sigma: float, lo: int, hi: int):
    def f(rng, n):
        x = np.exp(rng.normal(mu, sigma, size=n))
        return np.clip(np.rint(x), lo, hi).astype(np.int64)
    return f


WORKLOADS = {
    # tiny: batch 2, 8 query heads on 2 KV heads, head_dim 64, page 16, lengths 37 and 100,
    # 16-page pool, uniform[-1,1] values
    "tiny": dict(batch=2, query_heads=8, kv_heads=2, head_dim=64, page_size=16,
                 max_pages_per_sequence=8, context_lengths=[37, 100], pool_pages=16,
                 dist="uniform"),
    # small batch: 8 sequences of uniform length in [1, 4096], 2048-page pool
    "small_batch": dict(batch=8, query_heads=32, kv_heads=8, head_dim=128, page_size=16,
                        max_pages_per_sequence=256, ctx_sampler=_uniform_int(1, 4096),
                        pool_pages=2048, dist="normal"),
    # serving shaped: 64 sequences of uniform length in [512, 2048], pool +10% with holes
    "batch64": dict(batch=64, query_heads=32, kv_heads=8, head_dim=128, page_size=16,
                    max_pages_per_sequence=128, ctx_sampler=_uniform_int(512, 2048),
                    pool="holes10", dist="normal"),
    # long context: one 100000-token sequence, GQA 6, 1% of keys scaled x8, partition 1024
    "long100k": dict(batch=1, query_heads=24, kv_heads=4, head_dim=128, page_size=16,
                     max_pages_per_sequence=6250, context_lengths=[100000], pool="holes10",
                     dist="normal", outlier_fraction=0.01, outlier_factor=8.0,
                     partition_size=1024),
    # mixed large: 128 sequences, lognormal(7.5, 1) lengths clipped to [1, 32768], page 32
    "mixed128": dict(batch=128, query_heads=64, kv_heads=8, head_dim=128, page_size=32,
                     max_pages_per_sequence=1024,
                     ctx_sampler=_lognormal_clipped(7.5, 1.0, 1, 32768), pool="exact",
                     dist="normal"),
}

WORKLOAD_ORDER = ["tiny", "small_batch", "batch64", "long100k", "mixed128"]


def make_named(name: str, *, seed: Optional[int] = None, canary: bool = True) -> Workload:
    spec = dict(WORKLOADS[name])
    if seed is None:
        seed = 1000 + WORKLOAD_ORDER.index(name) + 1
    return make_workload(name=name, seed=seed, canary=canary, **spec)
