"""Pins that tie the CPU oracle to facts other than its own code.

Each ``pin_*`` takes an ``OracleUnderTest`` (the real oracle build, or a copy of
pa_oracle.c with a deliberately planted mistake) and raises AssertionError when
the oracle disagrees with:

* a library routine on a case that reduces to it (dense, non-paged attention via
  ``torch.softmax`` / ``torch.matmul`` in float64 on gathered K/V; numpy's own
  fp16 -> float64 conversion),
* a closed form (one token -> its value row; equal keys -> mean of values;
  two tokens -> the logistic mix),
* an invariant (physical-page relabelling is bitwise invisible; the result
  lies in the coordinate-wise hull of the value rows; linear in V),
* the split-context identity (per-partition (max, sum, acc) triples combined
  as in the V4 merge kernel of "[TIL] Optimizing paged attention" equal the
  direct evaluation).

The pins use small seeded inputs only (they run in the CPU suite).
"""
from __future__ import annotations

import math
import os

import numpy as np
import torch

from decode_attention_paged_03_amd import workloads as W
import oracle.pa_oracle as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


class OracleUnderTest:
    def __init__(self, lib_path=None):
        self.lib_path = lib_path

    def attend(self, wl, rows=None, nthreads=1, **over):
        a = dict(query=wl.query, key_cache=wl.key_cache, value_cache=wl.value_cache,
                 block_tables=wl.block_tables, context_lengths=wl.context_lengths,
                 scale=wl.scale)
        a.update(over)
        return O.attend(a["query"], a["key_cache"], a["value_cache"], a["block_tables"],
                        a["context_lengths"], a["scale"], rows=rows, nthreads=nthreads,
                        lib_path=self.lib_path)

    def attend_partitioned(self, wl, partition_size, rows=None, nthreads=1):
        return O.attend_partitioned(wl.query, wl.key_cache, wl.value_cache, wl.block_tables,
                                    wl.context_lengths, wl.scale, partition_size, rows=rows,
                                    nthreads=nthreads, lib_path=self.lib_path)

    def half(self, bits):
        return O.half_to_double(bits, lib_path=self.lib_path)

    def attend_zero_pages(self, wl, **over):
        a = dict(query=wl.query, key_cache=wl.key_cache, value_cache=wl.value_cache,
                 block_tables=wl.block_tables, context_lengths=wl.context_lengths,
                 scale=wl.scale)
        a.update(over)
        return O.attend(a["query"], a["key_cache"], a["value_cache"], a["block_tables"],
                        a["context_lengths"], a["scale"], lib_path=self.lib_path,
                        zero_pages=True)

    def bad_entries(self, bt, ctx, page_size, num_pages):
        return O.bad_entries(bt, ctx, page_size, num_pages, lib_path=self.lib_path)

    def append(self, new_k, new_v, bt, pos, k, v):
        return O.append(new_k, new_v, bt, pos, k, v, lib_path=self.lib_path)


# ----------------------------------------------------------------------------- helpers

def tiny(seed, *, B=2, QH=4, KVH=2, D=8, ps=4, ctx=None, max_pages=None, dist="normal",
         pool="holes10", scale=None, canary=True):
    if ctx is None:
        rng = np.random.default_rng(seed + 7)
        ctx = rng.integers(1, 40, size=B)
    return W.make_workload(name="pin", batch=B, query_heads=QH, kv_heads=KVH, head_dim=D,
                           page_size=ps, context_lengths=list(ctx),
                           max_pages_per_sequence=max_pages, pool=pool, dist=dist,
                           scale=scale, seed=seed, canary=canary)


def dense_reference(wl):
    """Non-paged attention with library routines: gather each sequence's K/V rows into a
    dense [L][KVH][D] array (numpy fancy indexing), broadcast KV heads to query heads with
    ``repeat_interleave`` and evaluate softmax(scale q K^T) V with torch in float64."""
    B, QH, KVH, D, ps = wl.batch, wl.query_heads, wl.kv_heads, wl.head_dim, wl.page_size
    G = QH // KVH
    kf = wl.key_cache.astype(np.float64).reshape(-1, KVH, D)
    vf = wl.value_cache.astype(np.float64).reshape(-1, KVH, D)
    out = np.zeros((B, QH, D))
    for b in range(B):
        L = int(wl.context_lengths[b])
        if L == 0:
            continue
        t = np.arange(L)
        rows = wl.block_tables[b, t // ps].astype(np.int64) * ps + t % ps
        K = torch.from_numpy(kf[rows]).repeat_interleave(G, dim=1)      # [L][QH][D]
        V = torch.from_numpy(vf[rows]).repeat_interleave(G, dim=1)
        q = torch.from_numpy(wl.query[b].astype(np.float64))            # [QH][D]
        s = torch.matmul(K.permute(1, 0, 2).contiguous(), q.unsqueeze(-1)).squeeze(-1) * wl.scale
        w = torch.softmax(s, dim=-1)                                      # [QH][L]
        out[b] = torch.matmul(w.unsqueeze(1), V.permute(1, 0, 2).contiguous()).squeeze(1).numpy()
    return out


def assert_close(a, b, rtol, atol=0.0, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    assert np.isfinite(a).all(), f"{what}: non-finite values"
    err = np.abs(a - b)
    bound = atol + rtol * np.abs(b)
    bad = err > bound
    assert not bad.any(), f"{what}: max err {err.max():.3e} at {np.argwhere(bad)[0]}"


def relabel_pages(wl, seed):
    """Move every physical page to a new index (a seeded permutation) and rewrite the
    block table to match: the same sequences, stored elsewhere in the pool."""
    rng = np.random.default_rng(seed)
    perm = rng.permutation(wl.num_pages)           # old index -> new index
    k = np.empty_like(wl.key_cache)
    v = np.empty_like(wl.value_cache)
    k[perm] = wl.key_cache
    v[perm] = wl.value_cache
    bt = wl.block_tables.copy()
    valid = bt >= 0
    bt[valid] = perm[bt[valid]]
    return k, v, bt


# ------------------------------------------------------------------------------- pins

def pin_half_exhaustive(ot):
    """All 65,536 binary16 patterns decode to numpy's float16 -> float64 value (NaN by class)."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([ot.half(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert (np.isnan(got) == nan).all(), "NaN classification differs"
    same = (got[~nan] == ref[~nan]) & (np.signbit(got[~nan]) == np.signbit(ref[~nan]))
    assert same.all(), f"first mismatch at bits {bits[~nan][~same][0]:#06x}"


def pin_dense_library(ot):
    """Paged oracle == dense torch-float64 attention on gathered rows, MHA/GQA/MQA shapes."""
    cases = [dict(B=3, QH=4, KVH=4, D=4, ps=4),      # MHA
             dict(B=2, QH=4, KVH=2, D=8, ps=4),      # GQA 2
             dict(B=3, QH=8, KVH=2, D=64, ps=8),     # GQA 4
             dict(B=2, QH=6, KVH=1, D=8, ps=2),      # MQA
             dict(B=1, QH=6, KVH=3, D=16, ps=16, dist="uniform")]
    for i, c in enumerate(cases):
        wl = tiny(100 + i, **c)
        assert_close(ot.attend(wl), dense_reference(wl), rtol=1e-12, atol=1e-14,
                     what=f"dense case {i}")


def pin_unpaged_identity(ot):
    """With the identity block table, sequence b's K/V are a plain reshape of its slab of
    the pool: no index arithmetic at all on the reference side."""
    B, QH, KVH, D, ps, mp = 3, 6, 2, 8, 4, 5
    wl = tiny(200, B=B, QH=QH, KVH=KVH, D=D, ps=ps, ctx=[20, 7, 13], max_pages=mp,
              pool="exact", canary=False)
    pool = np.random.default_rng(201).standard_normal((B * mp, ps, KVH, D)).astype(np.float16)
    poolv = np.random.default_rng(202).standard_normal((B * mp, ps, KVH, D)).astype(np.float16)
    bt = np.arange(B * mp, dtype=np.int32).reshape(B, mp)
    got = ot.attend(wl, key_cache=pool, value_cache=poolv, block_tables=bt)
    G = QH // KVH
    for b in range(B):
        L = int(wl.context_lengths[b])
        K = torch.from_numpy(pool[b * mp:(b + 1) * mp].reshape(mp * ps, KVH, D)[:L].astype(np.float64))
        V = torch.from_numpy(poolv[b * mp:(b + 1) * mp].reshape(mp * ps, KVH, D)[:L].astype(np.float64))
        for h in range(QH):
            q = torch.from_numpy(wl.query[b, h].astype(np.float64))
            w = torch.softmax(torch.mv(K[:, h // G, :].contiguous(), q) * wl.scale, dim=0)
            ref = torch.mv(V[:, h // G, :].t().contiguous(), w).numpy()
            assert_close(got[b, h], ref, rtol=1e-12, atol=1e-14, what=f"identity b{b} h{h}")


def pin_page_relabel_bitwise(ot):
    """Relabelling physical pages (and rewriting the table to match) changes no output bit."""
    wl = tiny(300, B=3, QH=8, KVH=2, D=16, ps=4, ctx=[33, 1, 18])
    a = ot.attend(wl)
    k, v, bt = relabel_pages(wl, 301)
    b = ot.attend(wl, key_cache=k, value_cache=v, block_tables=bt)
    assert np.array_equal(a.view(np.uint64), b.view(np.uint64)), "relabelling changed the output"


def pin_single_token(ot):
    """ctx = 1: the only weight is 1, so the output is that token's value row exactly."""
    wl = tiny(400, B=3, QH=4, KVH=2, D=8, ps=4, ctx=[1, 1, 1])
    out = ot.attend(wl)
    G = wl.group
    for b in range(wl.batch):
        phys = wl.block_tables[b, 0]
        for h in range(wl.query_heads):
            ref = wl.value_cache[phys, 0, h // G].astype(np.float64)
            assert np.array_equal(out[b, h], ref), f"b{b} h{h}"


def pin_equal_keys_mean(ot):
    """All keys equal (or q = 0): uniform weights, the output is the mean of the V rows."""
    wl = tiny(500, B=2, QH=4, KVH=2, D=8, ps=4, ctx=[11, 26])
    k = wl.key_cache.copy()
    k[:] = np.float16(0.375)
    q0 = np.zeros_like(wl.query)
    for over in (dict(key_cache=k), dict(query=q0)):
        out = ot.attend(wl, **over)
        G = wl.group
        for b in range(wl.batch):
            L = int(wl.context_lengths[b])
            t = np.arange(L)
            phys = wl.block_tables[b, t // wl.page_size]
            for h in range(wl.query_heads):
                rows = wl.value_cache[phys, t % wl.page_size, h // G].astype(np.float64)
                assert_close(out[b, h], rows.mean(0), rtol=1e-14, atol=1e-15, what="mean")


def pin_two_token_logistic(ot):
    """Two tokens with scores s0, s1: out = (v0 + e^(s1-s0) v1) / (1 + e^(s1-s0)).
    The dot products are small integers (exact in fp16 and double)."""
    D = 4
    q = np.array([[[1, 2, 0, 1]]], dtype=np.float16)                # B=1, QH=1
    k = np.zeros((1, 2, 1, D), dtype=np.float16)
    k[0, 0, 0] = [1, 0, 0, 0]                                       # q.k0 = 1
    k[0, 1, 0] = [0, 1, 3, 1]                                       # q.k1 = 3
    v = np.zeros((1, 2, 1, D), dtype=np.float16)
    v[0, 0, 0] = [1, -2, 0.5, 4]
    v[0, 1, 0] = [-1, 2, 0.25, 8]
    bt = np.zeros((1, 1), dtype=np.int32)
    for scale in (0.5, 1.0, 0.8125):
        got = O.attend(q, k, v, bt, np.array([2], np.int32), scale, lib_path=ot.lib_path)
        e = math.exp(scale * (3 - 1))
        ref = (v[0, 0, 0].astype(np.float64) + e * v[0, 1, 0].astype(np.float64)) / (1 + e)
        assert_close(got[0, 0], ref, rtol=1e-15, atol=1e-15, what=f"logistic scale={scale}")


def pin_hull_and_linearity(ot):
    """The output is a convex combination of V rows (coordinate-wise hull), and is linear
    in V for fixed q and K (V values chosen so that V1 + V2 is exact in fp16)."""
    wl = tiny(600, B=2, QH=4, KVH=2, D=8, ps=4, ctx=[17, 30], canary=False)
    rng = np.random.default_rng(601)
    v1 = (rng.integers(-64, 64, size=wl.value_cache.shape) / 16).astype(np.float16)
    v2 = (rng.integers(-64, 64, size=wl.value_cache.shape) / 16).astype(np.float16)
    o1 = ot.attend(wl, value_cache=v1)
    o2 = ot.attend(wl, value_cache=v2)
    o12 = ot.attend(wl, value_cache=(v1.astype(np.float32) + v2).astype(np.float16))
    assert_close(o12, o1 + o2, rtol=1e-12, atol=1e-12, what="linearity")
    G = wl.group
    for b in range(wl.batch):
        L = int(wl.context_lengths[b])
        t = np.arange(L)
        phys = wl.block_tables[b, t // wl.page_size]
        for h in range(wl.query_heads):
            rows = v1[phys, t % wl.page_size, h // G].astype(np.float64)
            assert (o1[b, h] >= rows.min(0) - 1e-12).all() and (o1[b, h] <= rows.max(0) + 1e-12).all()


def pin_large_shift(ot):
    """Scores near 2000 (exp would overflow double without the max shift): the oracle stays
    finite and agrees with torch's softmax, which shifts internally."""
    wl = tiny(700, B=2, QH=4, KVH=2, D=64, ps=8, ctx=[40, 23], scale=1.0, dist="uniform")
    q = np.full_like(wl.query, np.float16(4.0))
    k = wl.key_cache.copy()
    k[:, ::3] = np.float16(8.0)          # every third slot of every page: dot = 64*32 = 2048
    wl2 = W.Workload(**{**wl.__dict__, "query": q, "key_cache": k})
    assert_close(ot.attend(wl2), dense_reference(wl2), rtol=1e-11, atol=1e-13, what="large shift")


def pin_outlier_keys(ot):
    """Keys scaled x8 at 1% of positions (the long-context recipe, at a small size)."""
    wl = W.make_workload(name="pin", batch=1, query_heads=6, kv_heads=2, head_dim=16,
                         page_size=4, context_lengths=[300], pool="holes10", seed=800,
                         outlier_fraction=0.01, outlier_factor=8.0)
    assert_close(ot.attend(wl), dense_reference(wl), rtol=1e-12, atol=1e-14, what="outliers")


def pin_partition_identity(ot):
    """Per-partition (max, sum, acc) triples combined by the V4 merge rule equal the direct
    softmax, for partitions of one page, two pages, a non-multiple and one covering all."""
    wl = tiny(900, B=3, QH=6, KVH=3, D=8, ps=4, ctx=[37, 4, 61], max_pages=16)
    ref = ot.attend(wl)
    for part in (4, 8, 5, 64, 1024):
        assert_close(ot.attend_partitioned(wl, part), ref, rtol=1e-12, atol=1e-14,
                     what=f"partition {part}")


def pin_canaries_unread(ot):
    """NaN canaries in unreferenced pages and past-the-end slots never reach the output."""
    wl = tiny(1000, B=3, QH=4, KVH=2, D=8, ps=4, ctx=[5, 13, 2], canary=True)
    clean = tiny(1000, B=3, QH=4, KVH=2, D=8, ps=4, ctx=[5, 13, 2], canary=False)
    a = ot.attend(wl)
    b = ot.attend(clean)
    assert np.isfinite(a).all()
    assert np.array_equal(a, b)


def pin_layout_golden(ot):
    """The block-table picture of the Baseline section of "[TIL] Optimizing paged attention"
    (three streams on pages 0-2, 8-10 and 16-18 of a pool, 8 table slots each, the rest
    placeholders) evaluated against dense attention on the gathered rows."""
    import json
    with open(os.path.join(GOLDEN, "layout_example.json")) as f:
        fx = json.load(f)
    bt = np.array(fx["block_tables"], dtype=np.int32)
    B, mp = bt.shape
    ps, KVH, QH, D = fx["page_size"], fx["kv_heads"], fx["query_heads"], fx["head_dim"]
    ctx = np.array(fx["context_lengths"], dtype=np.int32)
    npages = fx["num_pages"]
    rng = np.random.default_rng(fx["seed"])
    wl = W.Workload(name="golden", batch=B, query_heads=QH, kv_heads=KVH, head_dim=D,
                    page_size=ps, max_pages_per_sequence=mp, num_pages=npages,
                    query=rng.standard_normal((B, QH, D)).astype(np.float16),
                    key_cache=rng.standard_normal((npages, ps, KVH, D)).astype(np.float16),
                    value_cache=rng.standard_normal((npages, ps, KVH, D)).astype(np.float16),
                    block_tables=bt, context_lengths=ctx, scale=0.25)
    assert_close(ot.attend(wl), dense_reference(wl), rtol=1e-12, atol=1e-14, what="layout")


def pin_errors_and_empty(ot):
    """ctx = 0 gives a zero row; an out-of-pool table entry or an over-long context is an
    error, not a read."""
    wl = tiny(1100, B=2, QH=4, KVH=2, D=8, ps=4, ctx=[0, 9])
    out = ot.attend(wl)
    assert np.array_equal(out[0], np.zeros_like(out[0]))
    bad = wl.block_tables.copy()
    bad[1, 1] = wl.num_pages
    for over in (dict(block_tables=bad),
                 dict(context_lengths=np.array([0, wl.max_pages_per_sequence * 4 + 1], np.int32))):
        try:
            ot.attend(wl, **over)
        except ValueError:
            continue
        raise AssertionError(f"no error for {list(over)}")


def _append_case(seed, B=5, KVH=3, D=8, ps=4, max_pages=4, num_pages=24):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((num_pages, ps, KVH, D)).astype(np.float16)
    v = rng.standard_normal((num_pages, ps, KVH, D)).astype(np.float16)
    owned = rng.permutation(num_pages)[:B * max_pages].reshape(B, max_pages).astype(np.int32)
    nk = rng.standard_normal((B, KVH, D)).astype(np.float16)
    nv = rng.standard_normal((B, KVH, D)).astype(np.float16)
    return k, v, owned, nk, nv


def pin_append_numpy_scatter(ot):
    """Storing a new token equals numpy's own scatter of the rows through the table
    (fancy-index assignment into the [pages][page_size][KVH][D] view), bit for bit, at
    positions on page boundaries, inside pages and at the table's last slot; a sequence
    with a negative position stores nothing."""
    for seed in range(3):
        k, v, bt, nk, nv = _append_case(1200 + seed)
        B, ps, mp = bt.shape[0], k.shape[1], bt.shape[1]
        pos = np.array([0, ps - 1, ps, mp * ps - 1, -1], dtype=np.int32)[:B]
        np.random.default_rng(seed).shuffle(pos)
        k2, v2, n = ot.append(nk, nv, bt, pos, k, v)
        live = pos >= 0
        ek, ev = k.copy(), v.copy()
        ek[bt[live, pos[live] // ps], pos[live] % ps] = nk[live]
        ev[bt[live, pos[live] // ps], pos[live] % ps] = nv[live]
        assert n == int(live.sum())
        assert np.array_equal(k2.view(np.uint16), ek.view(np.uint16)), "key cache"
        assert np.array_equal(v2.view(np.uint16), ev.view(np.uint16)), "value cache"


def pin_append_rebuilds_cache(ot):
    """Appending every token of a workload one decode step at a time, into a pool that
    starts as NaN canaries, rebuilds the workload's referenced cache rows exactly; the
    oracle's attention over the rebuilt cache is then bitwise the one over the original,
    and every slot no token reaches is still a canary."""
    wl = tiny(1300, B=3, QH=4, KVH=2, D=8, ps=4, ctx=[1, 9, 16])
    ps, KVH, D = wl.page_size, wl.kv_heads, wl.head_dim
    nan = np.full(wl.key_cache.shape, np.nan, dtype=np.float16)
    k, v = nan.copy(), nan.copy()
    kf = wl.key_cache.reshape(-1, KVH, D)
    vf = wl.value_cache.reshape(-1, KVH, D)
    ctx = wl.context_lengths
    for t in range(int(ctx.max())):
        pos = np.where(t < ctx, t, -1).astype(np.int32)
        rows = np.where(pos >= 0, wl.block_tables[np.arange(wl.batch), np.maximum(pos, 0) // ps]
                        .astype(np.int64) * ps + np.maximum(pos, 0) % ps, 0)
        k, v, n = ot.append(kf[rows], vf[rows], wl.block_tables, pos, k, v)
        assert n == int((pos >= 0).sum())
    assert np.array_equal(ot.attend(wl, key_cache=k, value_cache=v), ot.attend(wl))
    touched = np.zeros(wl.key_cache.shape[:2], dtype=bool)
    for b in range(wl.batch):
        t = np.arange(int(ctx[b]))
        touched[wl.block_tables[b, t // ps], t % ps] = True
    assert np.array_equal(k[touched].view(np.uint16), wl.key_cache[touched].view(np.uint16))
    assert np.array_equal(v[touched].view(np.uint16), wl.value_cache[touched].view(np.uint16))
    assert np.isnan(k[~touched]).all() and np.isnan(v[~touched]).all()


def pin_append_skips_unaddressable(ot):
    """A position past the table row or a table entry outside the pool stores nothing:
    the caches keep every old byte."""
    k, v, bt, nk, nv = _append_case(1400, B=3)
    ps, mp, npg = k.shape[1], bt.shape[1], k.shape[0]
    bad = bt.copy()
    bad[1, 0] = npg
    bad[2, 1] = -3
    pos = np.array([mp * ps, 1, ps + 2], dtype=np.int32)
    k2, v2, n = ot.append(nk, nv, bad, pos, k, v)
    assert n == 0
    assert np.array_equal(k2.view(np.uint16), k.view(np.uint16))
    assert np.array_equal(v2.view(np.uint16), v.view(np.uint16))


def plant_bad_entries(wl, seed, values):
    """A copy of wl's block table with entries outside the pool planted at chosen slots:
    (returns table, dereferenced slots, slots past the context).  Dereferenced slots are
    logical pages below ceil(ctx / page_size); the values cycle through ``values``."""
    rng = np.random.default_rng(seed)
    bt = wl.block_tables.copy()
    ps, mp = wl.page_size, wl.max_pages_per_sequence
    inside, past = [], []
    k = 0
    for b in range(wl.batch):
        n = (int(wl.context_lengths[b]) + ps - 1) // ps
        for lp in sorted(rng.choice(n, size=min(n, 2), replace=False)) if n else []:
            bt[b, lp] = values[k % len(values)]
            inside.append((b, int(lp)))
            k += 1
        if n < mp:
            bt[b, n] = values[k % len(values)]            # never dereferenced
            past.append((b, n))
            k += 1
    return bt, inside, past


def pin_zero_page_reading(ot):
    """Under the zero-page reading, a table entry outside the pool gives the same result,
    bit for bit, as the ordinary definition with that entry pointing at a real page of
    zeros appended to the pool; with no such entry both readings agree bitwise."""
    wl = tiny(1500, B=3, QH=4, KVH=2, D=8, ps=4, ctx=[9, 16, 5], max_pages=6, canary=False)
    assert np.array_equal(ot.attend_zero_pages(wl), ot.attend(wl))
    npg = wl.num_pages
    bt, inside, _ = plant_bad_entries(wl, 1501, [-1, npg, npg + 7, 2**31 - 1, -2**31])
    assert inside
    zk = np.concatenate([wl.key_cache, np.zeros_like(wl.key_cache[:1])])
    zv = np.concatenate([wl.value_cache, np.zeros_like(wl.value_cache[:1])])
    bt_zero = np.where((bt < 0) | (bt >= npg), npg, bt).astype(np.int32)
    got = ot.attend_zero_pages(wl, block_tables=bt)
    want = ot.attend(wl, block_tables=bt_zero, key_cache=zk, value_cache=zv)
    assert np.array_equal(got, want), "zero-page reading differs from a real zero page"
    assert not np.array_equal(got, ot.attend(wl)), "the planted entries changed nothing"


def pin_bad_entry_bitmap(ot):
    """The bitmap of bad entries holds exactly the planted dereferenced slots: not the
    planted slots past each context, and nothing for a clean table."""
    wl = tiny(1600, B=4, QH=4, KVH=2, D=8, ps=4, ctx=[9, 16, 1, 13], max_pages=7)
    mp, npg = wl.max_pages_per_sequence, wl.num_pages
    bitmap, n = ot.bad_entries(wl.block_tables, wl.context_lengths, wl.page_size, npg)
    assert n == 0 and not bitmap.any()
    bt, inside, past = plant_bad_entries(wl, 1601, [-1, npg, npg + 1, 2**31 - 1])
    bitmap, n = ot.bad_entries(bt, wl.context_lengths, wl.page_size, npg)
    bits = {i for i in range(wl.batch * mp) if (int(bitmap[i // 32]) >> (i % 32)) & 1}
    assert bits == {b * mp + lp for b, lp in inside}, (bits, inside, past)
    assert n == len(inside)


ALL_PINS = [pin_half_exhaustive, pin_dense_library, pin_unpaged_identity,
            pin_page_relabel_bitwise, pin_single_token, pin_equal_keys_mean,
            pin_two_token_logistic, pin_hull_and_linearity, pin_large_shift, pin_outlier_keys,
            pin_partition_identity, pin_canaries_unread, pin_layout_golden, pin_errors_and_empty,
            pin_append_numpy_scatter, pin_append_rebuilds_cache, pin_append_skips_unaddressable,
            pin_zero_page_reading, pin_bad_entry_bitmap]
