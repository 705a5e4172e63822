"""Block-table entries outside the pool.  Every call reads such an entry as a page of zero
keys and values (never dereferencing it); with PA_FLAG_DEBUG_BOUNDS the call also leaves
a bitmap of those entries at the start of the workspace.  Expected values come from the
oracle's zero-page reading and its bad-entry bitmap (both pinned on the CPU).  The
planted entries point at allocated NaN guard pages just before and after the pool, so a
read the clamp missed would poison the output rather than leave the allocation."""
import numpy as np
import pytest

from decode_attention_paged_03_amd import pa
from decode_attention_paged_03_amd import workloads as W

import gpu_common as C
from oracle_pins import plant_bad_entries

pytestmark = pytest.mark.gpu

GUARD_AFTER = 3


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pa.load()
    yield


def _case(shape, seed):
    QH, KVH, D, ps, ctx = shape
    wl = W.make_workload(name="bounds", batch=len(ctx), query_heads=QH, kv_heads=KVH, head_dim=D,
                         page_size=ps, context_lengths=ctx, pool="holes10", seed=seed,
                         max_pages_per_sequence=max(-(-c // ps) for c in ctx) + 2)
    npg = wl.num_pages
    # -1 lands on the guard page before the pool, npg .. npg + 2 on those after it
    bt, inside, past = plant_bad_entries(wl, seed + 1, [-1, npg, npg + 1, npg + GUARD_AFTER - 1])
    assert inside and max(bt.max(), npg) < npg + GUARD_AFTER
    return W.Workload(**{**wl.__dict__, "block_tables": bt}), inside


SHAPES = [
    (32, 8, 128, 16, [1, 40, 700, 2100, 5000, 17]),
    (24, 4, 128, 16, [3000, 16, 900]),
    (8, 2, 64, 8, [9, 100, 1031, 8]),          # tiles spanning two pages
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"qh{s[0]}_kvh{s[1]}_d{s[2]}_ps{s[3]}")
@pytest.mark.parametrize("route", ["balanced", "partition_4pages", "partition_1024"])
@pytest.mark.parametrize("debug", [False, True], ids=["clamp", "debug_bitmap"])
def test_out_of_pool_entries(shape, route, debug):
    import torch
    wl, inside = _case(shape, 7700 + SHAPES.index(shape) * 10)
    part = dict(balanced=0, partition_4pages=4 * wl.page_size, partition_1024=1024)[route]
    flags = pa.PA_FLAG_DEBUG_BOUNDS if debug else 0
    C.say(f"[case] out-of-pool entries {shape[:4]} route {route} debug {debug}: {len(inside)} planted")
    dev = C.Device(wl, guard=True, guard_after=GUARD_AFTER)
    dec = pa.decoder_for(wl, partition_size=part, flags=flags | C.fixed_flags(part))
    try:
        if dec.workspace is not None:
            dec.workspace.fill_(0xFF)        # every bitmap word must be written by the call
        out = dev.run(dec).cpu().numpy()
        ref = C.oracle.attend(wl.query, wl.key_cache, wl.value_cache, wl.block_tables,
                              wl.context_lengths, wl.scale, nthreads=C.oracle_threads(),
                              zero_pages=True)
        C.check_against_oracle(out, ref, f"zero pages {route} debug={debug}")
        if debug:
            want, n = C.oracle.bad_entries(wl.block_tables, wl.context_lengths, wl.page_size,
                                           wl.num_pages)
            assert n == len(inside)
            got = dec.bad_entry_bitmap()
            assert np.array_equal(got, want), f"bitmap {got} != {want}"
    finally:
        dec.close()


def test_clean_table_bitmap_empty_and_output_unchanged():
    """A table with every entry in the pool: an all-zero bitmap, and the same output bits
    as without the flag."""
    import torch
    wl = W.make_named("small_batch")
    dev = C.Device(wl)
    outs = []
    for flags in (0, pa.PA_FLAG_DEBUG_BOUNDS):
        dec = pa.decoder_for(wl, partition_size=0, flags=flags)
        try:
            if dec.workspace is not None:
                dec.workspace.fill_(0xFF)
            outs.append(dev.run(dec).clone())
            if flags:
                assert not dec.bad_entry_bitmap().any()
        finally:
            dec.close()
    assert torch.equal(outs[0].view(torch.int32), outs[1].view(torch.int32))
