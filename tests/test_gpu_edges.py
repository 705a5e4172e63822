"""GPU edge cases of pa_decode beyond the workload and shape sweeps: the scale's sign and
zero, a workspace full of garbage before the call, the fallback of very large batches
to fixed partitions, and an explicit max_context_length.  Same bar as the parity tests:
|gpu - oracle| <= 1e-3 * (1 + |oracle|), with NaN canaries never read."""
import numpy as np
import pytest

from decode_attention_paged_03_amd import pa
from decode_attention_paged_03_amd import workloads as W

import gpu_common as C

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pa.load()
    yield


def _small(seed, scale=None, **kw):
    d = dict(name="edge", batch=4, query_heads=16, kv_heads=4, head_dim=128, page_size=16,
             context_lengths=[1, 700, 2100, 33], pool="holes10", seed=seed, scale=scale)
    d.update(kw)
    return W.make_workload(**d)


@pytest.mark.parametrize("scale", [-1.0 / np.sqrt(128), 0.0, 0.35])
@pytest.mark.parametrize("partition", [0, 256])
def test_scale_sign_and_zero(scale, partition):
    """A negative scale is folded into q as a sign flip; scale 0 gives the plain mean of
    the value rows; a large scale sharpens the weights."""
    wl = _small(7300, scale=scale, partition_size=partition)
    C.decode_and_check(wl, what=f"scale {scale:+.4f} partition {partition}")


@pytest.mark.parametrize("partition", [0, 128])
def test_workspace_garbage_ignored(partition):
    """Workspace bytes left by anything else (here all 0xFF: NaN floats, -1 integers) do
    not reach the output: every value the merge reads is written by the same call."""
    import torch
    wl = W.make_named("small_batch")
    C.say(f"[case] garbage workspace, partition {partition}")
    dev = C.Device(wl)
    dec = pa.decoder_for(wl, partition_size=partition, flags=C.fixed_flags(partition))
    try:
        assert dec.workspace is not None
        dec.workspace.fill_(0xFF)
        out = dev.run(dec).cpu().numpy()
    finally:
        dec.close()
    C.check_against_oracle(out, C.oracle.attend_workload(wl, nthreads=C.oracle_threads()),
                           f"garbage workspace partition {partition}")


def test_workspace_shared_by_two_problems():
    """One workspace buffer serves two different problems in turn (a long single
    sequence, then a batch); the second result is unaffected by the first's leftovers."""
    import torch
    long_wl = W.make_workload(name="ws_long", batch=1, query_heads=24, kv_heads=4,
                              head_dim=128, page_size=16, context_lengths=[20000],
                              pool="holes10", seed=7400)
    batch_wl = W.make_workload(name="ws_batch", batch=24, query_heads=32, kv_heads=8,
                               head_dim=128, page_size=16,
                               context_lengths=list(range(40, 24 * 97, 97)),
                               pool="holes10", seed=7401)
    decs = [pa.decoder_for(w) for w in (long_wl, batch_wl)]
    try:
        need = max(d.workspace_bytes for d in decs)
        ws = torch.full((need,), 0x7F, dtype=torch.uint8, device="cuda")
        outs = []
        for wl_, dec in zip((long_wl, batch_wl), decs):
            C.say(f"[case] shared workspace: {wl_.summary()}")
            dev = C.Device(wl_)
            out = torch.full((wl_.batch, wl_.query_heads, wl_.head_dim), float("nan"),
                             device="cuda")
            stream = torch.cuda.current_stream()
            pa.pa_decode(dec.handle, dev.q.data_ptr(), dev.k.data_ptr(), dev.v.data_ptr(),
                         dev.bt.data_ptr(), dev.ctx.data_ptr(), wl_.scale, out.data_ptr(),
                         ws.data_ptr(), need, stream.cuda_stream)
            torch.cuda.synchronize()
            outs.append(out.cpu().numpy())
        for wl_, out in zip((long_wl, batch_wl), outs):
            C.check_against_oracle(out, C.oracle.attend_workload(wl_, nthreads=C.oracle_threads()),
                                   f"shared workspace {wl_.name}")
    finally:
        for d in decs:
            d.close()


def test_large_batch_falls_back_to_partitions():
    """More sequences than the balanced route keeps in LDS (2048): the library uses fixed
    partitions of the default size, with and without single-pass sequences."""
    rng = np.random.default_rng(7500)
    ctx = rng.integers(0, 60, size=2100)
    ctx[::97] = 1500                              # a few sequences that need two partitions
    wl = W.make_workload(name="big_batch", batch=2100, query_heads=8, kv_heads=2, head_dim=64,
                         page_size=16, context_lengths=list(ctx), pool="holes10", seed=7501)
    dec = pa.decoder_for(wl)
    try:
        assert dec.workspace_bytes > 0            # fixed partitions of 1024 with a merge
    finally:
        dec.close()
    C.decode_and_check(wl, what="batch 2100")


@pytest.mark.parametrize("partition", [0, 64])
def test_max_context_length_bound(partition):
    """max_context_length set to the longest sequence (smaller than the table allows):
    the grid and workspace are sized from it, and every length up to it is handled."""
    import torch
    wl = W.make_workload(name="maxctx", batch=5, query_heads=8, kv_heads=2, head_dim=128,
                         page_size=16, context_lengths=[0, 17, 500, 999, 1000],
                         max_pages_per_sequence=200, pool="holes10", seed=7600)
    C.say(f"[case] max_context_length 1000 (table allows {200 * 16}), partition {partition}")
    dev = C.Device(wl)
    dec = pa.decoder_for(wl, partition_size=partition, max_context_length=1000,
                         flags=C.fixed_flags(partition))
    try:
        out = dev.run(dec).cpu().numpy()
    finally:
        dec.close()
    C.check_against_oracle(out, C.oracle.attend_workload(wl, nthreads=C.oracle_threads()),
                           f"max_context_length partition {partition}")


def test_concurrent_streams_distinct_workspaces():
    """Two calls in flight at once on two streams, each with its own handle and workspace
    (the documented rule for concurrency), give the same bits as the calls made one after
    the other."""
    import torch
    wls = [W.make_named("small_batch"), W.make_named("tiny")]
    devs = [C.Device(w) for w in wls]
    decs = [pa.decoder_for(w) for w in wls]
    try:
        ref = [dev.run(dec).clone() for dev, dec in zip(devs, decs)]
        streams = [torch.cuda.Stream(), torch.cuda.Stream()]
        outs = [torch.full_like(r, float("nan")) for r in ref]
        torch.cuda.synchronize()
        for _ in range(3):
            for wl_, dev, dec, s, out in zip(wls, devs, decs, streams, outs):
                dec(dev.q, dev.k, dev.v, dev.bt, dev.ctx, wl_.scale, out=out, stream=s)
        torch.cuda.synchronize()
        for r, out in zip(ref, outs):
            assert torch.equal(r.view(torch.int32), out.view(torch.int32))
    finally:
        for d in decs:
            d.close()


@pytest.mark.parametrize("batch", [96, 1500])
def test_eight_heads_per_wave_both_k_layouts(batch):
    """Eight query heads per wave: with a moderate batch the kernel stages K rows through
    LDS; with 1500 sequences the per-sequence arrays leave no room for that staging and
    K is loaded in the MFMA layout instead.  Both agree with the oracle."""
    rng = np.random.default_rng(7700 + batch)
    ctx = rng.integers(1, 300, size=batch)
    wl = W.make_workload(name="g8", batch=batch, query_heads=16, kv_heads=2, head_dim=128,
                         page_size=16, context_lengths=list(ctx), pool="holes10",
                         seed=7701 + batch)
    C.decode_and_check(wl, what=f"8 heads per wave, batch {batch}")
