"""GPU parity of pa_append (HIP, through the C ABI) against the CPU oracle's append.

Storing rows is byte work, so the bar is bit-exact: after the call both caches, guard
page included, must equal the oracle's caches byte for byte.  The decode-loop test then
stores a sequence's newest tokens one step at a time and checks each step's pa_decode
against the oracle's attention over the same context (the usual 1e-3 * (1 + |oracle|)).
"""
import numpy as np
import pytest

from decode_attention_paged_03_amd import pa
from decode_attention_paged_03_amd import workloads as W

import gpu_common as C
import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pa.load()
    yield


def _new_rows(wl, seed):
    rng = np.random.default_rng(seed)
    shape = (wl.batch, wl.kv_heads, wl.head_dim)
    return (rng.standard_normal(shape).astype(np.float16),
            rng.standard_normal(shape).astype(np.float16))


def _append_and_compare(wl, positions, block_tables=None, what=""):
    import torch
    bt = wl.block_tables if block_tables is None else block_tables
    pos = np.asarray(positions, dtype=np.int32)
    nk, nv = _new_rows(wl, 77 + wl.batch)
    C.say(f"[case] append {what}: {wl.summary()} positions[:8]={pos[:8].tolist()}")
    dev = C.Device(wl)
    dec = pa.decoder_for(wl)
    try:
        dec.append(torch.from_numpy(nk).cuda(), torch.from_numpy(nv).cuda(), dev.k, dev.v,
                   torch.from_numpy(np.ascontiguousarray(bt)).cuda(),
                   torch.from_numpy(pos).cuda())
        torch.cuda.synchronize()
    finally:
        dec.close()
    ek, ev, n = oracle.append(nk, nv, bt, pos, wl.key_cache, wl.value_cache)
    for name, alloc, exp in (("key", dev.k_alloc, ek), ("value", dev.v_alloc, ev)):
        got = alloc.cpu().numpy().view(np.uint16)
        assert np.isnan(got[0].view(np.float16)).all(), f"{name}: guard page written"
        diff = got[1:] != exp.view(np.uint16)
        assert not diff.any(), f"{name}: {int(diff.sum())} elements differ, first {np.argwhere(diff)[0]}"
    C.say(f"[append] {what}: {n} sequences stored, caches bit-exact")
    return n


@pytest.mark.parametrize("QH,KVH,D,ps", [(32, 8, 128, 16), (8, 2, 64, 8), (24, 4, 128, 32),
                                         (8, 1, 128, 256)])
def test_append_edges(QH, KVH, D, ps):
    """Positions on page boundaries, inside pages, at the table's last slot, negative,
    past the table, and through table entries outside the pool (skipped)."""
    B, mp = 12, 6
    ctx = [1, ps - 1, ps, ps + 1, 2 * ps, mp * ps, 3, 5, ps * 2 + 3, 7, 9, 11]
    wl = W.make_workload(name="append_edges", batch=B, query_heads=QH, kv_heads=KVH,
                         head_dim=D, page_size=ps, context_lengths=ctx,
                         max_pages_per_sequence=mp, pool="holes10", dist="normal",
                         seed=3100 + ps, canary=True)
    bt = wl.block_tables.copy()
    # every sequence owns all of its table row's pages (the generator leaves -1 past ctx)
    free = [p for p in range(wl.num_pages) if p not in set(bt[bt >= 0].tolist())]
    pos = np.array([c - 1 for c in ctx], dtype=np.int32)   # rewrite each sequence's last row
    pos[1] = ps - 1
    pos[2] = ps                                             # first slot of a page not yet in use
    pos[3] = ps + 1
    pos[5] = mp * ps - 1                                    # last slot of the table row
    pos[6] = -1                                             # nothing to store
    pos[7] = mp * ps                                        # past the table: skipped
    pos[9] = 2 * ps                                         # table entry made out of pool below
    pos[10] = ps                                            # table entry made negative below
    for b, p in ((2, 1), (3, 1)):
        if bt[b, p] < 0:
            bt[b, p] = free.pop()
    bt[9, 2] = wl.num_pages
    bt[10, 1] = -5
    n = _append_and_compare(wl, pos, bt, what=f"edges QH{QH}/KVH{KVH} D{D} ps{ps}")
    assert n == B - 4


def test_append_batch64_full():
    """The 64-sequence decode workload at full size: each sequence stores its newest row
    (the slot of its last cached token), bit-exact against the oracle on the whole pool."""
    wl = W.make_named("batch64")
    _append_and_compare(wl, wl.context_lengths - 1, what="batch64")


def test_append_then_decode_steps():
    """A decode loop: the cache starts without each sequence's last three tokens (their
    slots hold NaN canaries); three steps each store one token with pa_append and attend
    with pa_decode over context position + 1.  Every step matches the oracle's attention
    over the original workload truncated to the same lengths, and after the last step the
    caches equal the original bit for bit."""
    import torch
    wl = W.make_named("small_batch")
    ps, KVH, D = wl.page_size, wl.kv_heads, wl.head_dim
    ctx = wl.context_lengths.astype(np.int64)
    steps = 3
    start = np.maximum(ctx - steps, 0)
    kf = wl.key_cache.reshape(-1, KVH, D)
    vf = wl.value_cache.reshape(-1, KVH, D)
    k0, v0 = wl.key_cache.copy(), wl.value_cache.copy()
    for b in range(wl.batch):
        for t in range(int(start[b]), int(ctx[b])):
            page, slot = wl.block_tables[b, t // ps], t % ps
            k0[page, slot] = np.nan
            v0[page, slot] = np.nan
    dev = C.Device(wl)
    dev.k.copy_(torch.from_numpy(k0))
    dev.v.copy_(torch.from_numpy(v0))
    dec = pa.decoder_for(wl)
    try:
        for s in range(steps):
            pos = start + s
            live = pos < ctx
            posv = np.where(live, pos, -1).astype(np.int32)
            rows = np.where(live, wl.block_tables[np.arange(wl.batch),
                                                  np.minimum(pos, ctx - 1) // ps].astype(np.int64)
                            * ps + np.minimum(pos, ctx - 1) % ps, 0)
            C.say(f"[case] decode step {s}: positions {posv.tolist()}")
            dec.append(torch.from_numpy(np.ascontiguousarray(kf[rows])).cuda(),
                       torch.from_numpy(np.ascontiguousarray(vf[rows])).cuda(),
                       dev.k, dev.v, dev.bt, torch.from_numpy(posv).cuda())
            lens = np.where(live, pos + 1, np.minimum(ctx, start + steps)).astype(np.int32)
            out = torch.full((wl.batch, wl.query_heads, D), float("nan"), device="cuda")
            dec(dev.q, dev.k, dev.v, dev.bt, torch.from_numpy(lens).cuda(), wl.scale, out=out)
            torch.cuda.synchronize()
            ref = oracle.attend(wl.query, wl.key_cache, wl.value_cache, wl.block_tables, lens,
                                wl.scale, nthreads=C.oracle_threads())
            C.check_against_oracle(out.cpu().numpy(), ref, f"decode step {s}")
    finally:
        dec.close()
    assert np.array_equal(dev.k.cpu().numpy().view(np.uint16), wl.key_cache.view(np.uint16))
    assert np.array_equal(dev.v.cpu().numpy().view(np.uint16), wl.value_cache.view(np.uint16))
