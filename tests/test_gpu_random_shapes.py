"""Seeded random problem shapes against the oracle: through the library's own route (the
balanced split, or one partition per sequence for short contexts), fixed partitions, the
single launch and the bounds-checking flag.

Each case draws a batch size, a head layout (KV heads and group size, hence heads per wave
and streams per sequence), a head dimension, a page size and a mix of context lengths
(zeros, single tokens, a long sequence among short ones, runs of equal lengths), so that
the split, the stream bands, the merge paths and the sequence search meet shapes no
fixed list names.  The draws are seeded: every run checks the same cases.

Bar: |gpu - oracle| <= 1e-3 * (1 + |oracle|), with NaN canaries never read.
"""
import numpy as np
import pytest

from decode_attention_paged_03_amd import pa
from decode_attention_paged_03_amd import workloads as W

import gpu_common as C

pytestmark = pytest.mark.gpu

N_CASES = 24


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pa.load()
    yield


def _draw(seed):
    rng = np.random.default_rng(seed)
    kv_heads = int(rng.choice([1, 2, 3, 4, 8]))
    group = int(rng.choice([1, 2, 3, 4, 5, 6, 8, 12, 16]))
    head_dim = int(rng.choice([64, 128]))
    page_size = int(rng.choice([8, 16, 32, 64, 128, 256]))
    batch = int(rng.integers(1, 48))
    kind = rng.integers(0, 4)
    if kind == 0:                                   # uniform lengths
        ctx = rng.integers(0, 3000, size=batch)
    elif kind == 1:                                 # lognormal, clipped
        ctx = np.clip(rng.lognormal(6.0, 1.2, size=batch), 1, 6000).astype(np.int64)
    elif kind == 2:                                 # one long sequence among short ones
        ctx = rng.integers(0, 40, size=batch)
        ctx[rng.integers(0, batch)] = int(rng.integers(8000, 30000))
    else:                                           # runs of equal lengths
        ctx = np.repeat(rng.integers(1, 700, size=(batch + 3) // 4), 4)[:batch]
    ctx[rng.random(batch) < 0.1] = 0                # some empty sequences
    ctx[rng.random(batch) < 0.1] = 1                # some single tokens
    # keep the oracle's work bounded (about 60 K tokens per case)
    total = int(ctx.sum())
    if total > 60000:
        ctx = (ctx * (60000 / total)).astype(np.int64)
    return dict(batch=batch, query_heads=kv_heads * group, kv_heads=kv_heads,
                head_dim=head_dim, page_size=page_size, context_lengths=[int(c) for c in ctx])


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_shape(case):
    d = _draw(9900 + case)
    wl = W.make_workload(name=f"random{case}", pool="holes10", seed=9950 + case, **d)
    C.decode_and_check(wl, what=f"random case {case}: QH{d['query_heads']}/KVH{d['kv_heads']} "
                                f"D{d['head_dim']} ps{d['page_size']} B{d['batch']}")


@pytest.mark.parametrize("case", range(0, N_CASES, 2))
def test_random_shape_fixed_partitions(case):
    """The same draws through the fixed-partition route, with a partition of 1, 2, 4 or 16
    pages."""
    d = _draw(9900 + case)
    pages = [1, 2, 4, 16][case // 2 % 4]
    wl = W.make_workload(name=f"random{case}", pool="holes10", seed=9950 + case, **d)
    C.decode_and_check(wl, partition_size=pages * d["page_size"],
                       what=f"random case {case}, partition of {pages} pages")


@pytest.mark.parametrize("case", range(1, N_CASES, 2))
def test_random_shape_single_launch(case):
    """The same draws with the merge folded into the decode launch (PA_FLAG_SINGLE_LAUNCH):
    bands crossing workgroups of every span the draws give."""
    d = _draw(9900 + case)
    wl = W.make_workload(name=f"random{case}", pool="holes10", seed=9950 + case, **d)
    C.decode_and_check(wl, partition_size=0, flags=pa.PA_FLAG_SINGLE_LAUNCH,
                       what=f"random case {case}, single launch")


@pytest.mark.parametrize("case", range(0, N_CASES, 3))
def test_random_shape_debug_bounds(case):
    """PA_FLAG_DEBUG_BOUNDS on valid tables: the output is unchanged and the bitmap of
    out-of-pool entries equals the oracle's (all clear)."""
    import torch
    d = _draw(9900 + case)
    wl = W.make_workload(name=f"random{case}", pool="holes10", seed=9950 + case, **d)
    C.say(f"[case] random case {case}, debug bounds: {wl.summary()}")
    dev = C.Device(wl)
    plain = pa.decoder_for(wl, partition_size=0)
    dbg = pa.decoder_for(wl, partition_size=0, flags=pa.PA_FLAG_DEBUG_BOUNDS)
    try:
        want = dev.run(plain).clone()
        got = dev.run(dbg).clone()
        torch.cuda.synchronize()
        assert torch.equal(want.view(torch.int32), got.view(torch.int32))
        bitmap = dbg.bad_entry_bitmap()
    finally:
        plain.close()
        dbg.close()
    exp_bitmap, count = C.oracle.bad_entries(wl.block_tables, wl.context_lengths, wl.page_size,
                                             wl.num_pages)
    assert count == 0
    assert np.array_equal(bitmap[:len(exp_bitmap)], np.asarray(exp_bitmap, dtype=np.uint32))


def _draw_short(seed):
    """A shape whose bands are all short enough for one partition per sequence: heads per
    wave, streams and streams per band as the plan derives them, contexts up to the
    longest band that mode takes (24 stream tiles), with empty sequences and single
    tokens among them."""
    import math
    rng = np.random.default_rng(seed)
    kv_heads = int(rng.choice([1, 2, 3, 4, 8]))
    group = int(rng.choice([1, 2, 3, 4, 6, 8]))
    hp = max(h for h in range(1, 9) if group % h == 0)
    streams = kv_heads * (group // hp)
    batch = int(rng.integers(1, 40))
    spw = math.gcd(streams, 12)
    if batch * (streams // spw) < 32 and spw % 2 == 0:
        spw //= 2
    page_size = int(rng.choice([8, 16, 32]))
    cap = 16 * (24 // spw)                      # tokens: the longest band of this mode
    longest = (cap // page_size) * page_size   # the table's bound must fit it too
    ctx = rng.integers(0, longest + 1, size=batch)
    ctx[rng.random(batch) < 0.15] = 1
    ctx[rng.random(batch) < 0.15] = 0
    ctx[int(rng.integers(0, batch))] = longest
    return dict(batch=batch, query_heads=kv_heads * group, kv_heads=kv_heads,
                head_dim=int(rng.choice([64, 128])), page_size=page_size,
                context_lengths=[int(c) for c in ctx])


@pytest.mark.parametrize("case", range(16))
def test_random_short_contexts(case):
    """Seeded shapes with short contexts only, which take one partition per sequence (the
    fixed kernel, 8 or 4 waves): up to 24 tiles per band, empty sequences and single
    tokens, pages of 8 to 32."""
    d = _draw_short(9700 + case)
    wl = W.make_workload(name=f"short{case}", pool="holes10", seed=9750 + case, **d)
    dec = pa.decoder_for(wl, partition_size=0)
    try:
        assert dec.workspace_bytes == 0, f"case {case}: expected one partition per sequence ({d})"
    finally:
        dec.close()
    C.decode_and_check(wl, partition_size=0,
                       what=f"short contexts case {case}: QH{d['query_heads']}/KVH{d['kv_heads']} "
                            f"D{d['head_dim']} ps{d['page_size']} B{d['batch']}")


def _draw_wide_short(seed):
    """A shape for the other short-context rule: at least 64 workgroups (sequences x KV
    heads x head chunks) and the longest sequence within 8 tiles per wave (1024 tokens
    with 8 waves when the grid fits 256 compute units, 512 with 4), with empty sequences
    and single tokens among them."""
    import math
    rng = np.random.default_rng(seed)
    kv_heads = int(rng.choice([2, 4, 8]))
    group = int(rng.choice([1, 2, 4, 6, 8, 16]))
    hp = max(h for h in range(1, 9) if group % h == 0)
    per_seq = kv_heads * (group // hp)
    lo = math.ceil(64 / per_seq)
    batch = int(rng.integers(lo, max(lo + 1, 600 // per_seq + 1)))
    waves = 8 if batch * per_seq <= 256 else 4
    page_size = int(rng.choice([8, 16, 32]))
    longest = 16 * 8 * waves // page_size * page_size
    ctx = rng.integers(0, longest + 1, size=batch)
    ctx[rng.random(batch) < 0.1] = 0
    ctx[rng.random(batch) < 0.1] = 1
    # keep the oracle's work bounded (about 40 M token-heads per case)
    if int(ctx.sum()) * kv_heads * group > 40_000_000:
        ctx = (ctx * (40_000_000 / (int(ctx.sum()) * kv_heads * group))).astype(np.int64)
    ctx[int(rng.integers(0, batch))] = longest
    return dict(batch=batch, query_heads=kv_heads * group, kv_heads=kv_heads,
                head_dim=int(rng.choice([64, 128])), page_size=page_size,
                context_lengths=[int(c) for c in ctx])


@pytest.mark.parametrize("case", range(12))
def test_random_wide_short_contexts(case):
    """Seeded shapes of many short sequences (at least 64 workgroups, at most 8 tiles per
    wave), which also take one partition per sequence, on grids both within and beyond
    the compute units (8 and 4 waves per workgroup)."""
    d = _draw_wide_short(9800 + case)
    wl = W.make_workload(name=f"wide_short{case}", pool="holes10", seed=9850 + case, **d)
    dec = pa.decoder_for(wl, partition_size=0)
    try:
        assert dec.workspace_bytes == 0, f"case {case}: expected one partition per sequence ({d})"
    finally:
        dec.close()
    C.decode_and_check(wl, partition_size=0,
                       what=f"wide short contexts case {case}: QH{d['query_heads']}/KVH{d['kv_heads']} "
                            f"D{d['head_dim']} ps{d['page_size']} B{d['batch']}")
