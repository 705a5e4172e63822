"""The C ABI on the host: the library loads, exports what include/pa.h declares, and
rejects bad arguments before any HIP call (no GPU needed)."""
import ctypes
import os
import re
import subprocess

import pytest

from decode_attention_paged_03_amd import pa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pa.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pa.LIB_PATH):
        from decode_attention_paged_03_amd import build
        build.build()
    return pa.load()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(pa_\w+)\s*\(", text, re.M)))


def test_header_declares_the_abi():
    assert declared_functions() == sorted(pa.EXPORTED)


def test_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", pa.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    syms = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in declared_functions():
        assert name in syms, name
        assert getattr(lib, name) is not None


def good(**over):
    d = dict(batch=2, query_heads=8, kv_heads=2, head_dim=128, page_size=16,
             max_pages_per_sequence=8, num_physical_pages=16, partition_size=0,
             max_context_length=0, flags=0)
    d.update(over)
    return pa.make_problem(**d)


def create_status(prob):
    h = ctypes.c_void_p()
    st = pa.load().pa_create(ctypes.byref(prob), ctypes.byref(h))
    if st == pa.PA_OK:
        pa.pa_destroy(h)
    else:
        assert not h.value
    return st


@pytest.mark.parametrize("over,status", [
    ({}, pa.PA_OK),
    (dict(head_dim=64), pa.PA_OK),
    (dict(batch=0), pa.PA_ERR_INVALID_ARGUMENT),
    (dict(query_heads=6, kv_heads=4), pa.PA_ERR_INVALID_ARGUMENT),
    (dict(kv_heads=0), pa.PA_ERR_INVALID_ARGUMENT),
    (dict(head_dim=96), pa.PA_ERR_UNSUPPORTED),
    (dict(head_dim=-1), pa.PA_ERR_INVALID_ARGUMENT),
    (dict(page_size=12), pa.PA_ERR_UNSUPPORTED),
    (dict(page_size=4), pa.PA_ERR_UNSUPPORTED),
    (dict(page_size=512), pa.PA_ERR_UNSUPPORTED),
    (dict(page_size=0), pa.PA_ERR_INVALID_ARGUMENT),
    (dict(max_pages_per_sequence=0), pa.PA_ERR_INVALID_ARGUMENT),
    (dict(num_physical_pages=0), pa.PA_ERR_INVALID_ARGUMENT),
    (dict(partition_size=24), pa.PA_ERR_INVALID_ARGUMENT),
    (dict(partition_size=-16), pa.PA_ERR_INVALID_ARGUMENT),
    (dict(partition_size=16 * 513), pa.PA_ERR_UNSUPPORTED),
    (dict(max_context_length=8 * 16 + 1), pa.PA_ERR_INVALID_ARGUMENT),
    (dict(flags=0x100), pa.PA_ERR_INVALID_ARGUMENT),
    (dict(flags=0x20), pa.PA_ERR_INVALID_ARGUMENT),
    (dict(flags=pa.PA_FLAG_FIXED_PARTITIONS, partition_size=16), pa.PA_OK),
    (dict(flags=pa.PA_FLAG_FIXED_PARTITIONS | pa.PA_FLAG_SINGLE_LAUNCH), pa.PA_ERR_INVALID_ARGUMENT),
    (dict(flags=pa.PA_FLAG_DEBUG_BOUNDS), pa.PA_OK),
    (dict(flags=pa.PA_FLAG_DEBUG_BOUNDS | pa.PA_FLAG_FORCE_SPLIT), pa.PA_OK),
    (dict(flags=pa.PA_FLAG_SINGLE_LAUNCH), pa.PA_OK),
    (dict(flags=pa.PA_FLAG_SINGLE_LAUNCH | pa.PA_FLAG_DEBUG_BOUNDS), pa.PA_OK),
    (dict(flags=pa.PA_FLAG_SINGLE_LAUNCH, partition_size=16), pa.PA_ERR_INVALID_ARGUMENT),
    (dict(flags=pa.PA_FLAG_SINGLE_LAUNCH | pa.PA_FLAG_FORCE_SPLIT), pa.PA_ERR_INVALID_ARGUMENT),
    (dict(flags=pa.PA_FLAG_SINGLE_LAUNCH, batch=4096, max_pages_per_sequence=1,
          num_physical_pages=4096), pa.PA_ERR_UNSUPPORTED),
    (dict(flags=pa.PA_FLAG_FORCE_SPLIT | pa.PA_FLAG_FORCE_SINGLE), pa.PA_ERR_INVALID_ARGUMENT),
    (dict(flags=pa.PA_FLAG_FORCE_SINGLE, max_pages_per_sequence=4096), pa.PA_ERR_UNSUPPORTED),
])
def test_create_validation(lib, over, status):
    assert create_status(good(**over)) == status


def test_create_null_arguments(lib):
    h = ctypes.c_void_p()
    assert lib.pa_create(None, ctypes.byref(h)) == pa.PA_ERR_INVALID_ARGUMENT
    prob = good()
    assert lib.pa_create(ctypes.byref(prob), None) == pa.PA_ERR_INVALID_ARGUMENT
    assert lib.pa_destroy(None) == pa.PA_OK


def ws_size(**over):
    h = pa.pa_create(good(**over))
    try:
        return pa.pa_workspace_size(h)
    finally:
        pa.pa_destroy(h)


def test_workspace_size():
    # no partition size, no flag: balanced route.  Per workgroup (up to 1024): two sides x
    # the streams read side by side x heads_per_wg rows of (D + 2) floats, plus two 16-byte
    # records.  Streams side by side: gcd(streams, 12), halved while the batch holds fewer
    # than 32 bands.  Group 4 -> 4 heads per wave; 2 KV heads, batch 2 -> 2 bands -> 1.
    # (A table of 128 pages: sequences longer than the one-partition-per-sequence limit.)
    L = dict(max_pages_per_sequence=128, num_physical_pages=512)
    assert ws_size(**L) == 1024 * 2 * 1 * 4 * (128 + 2) * 4 + 1024 * 32
    # 32 sequences: 32 bands of 2 streams, kept side by side
    assert ws_size(batch=32, **L) == 1024 * 2 * 2 * 4 * (128 + 2) * 4 + 1024 * 32
    # 4 KV heads (group 6 -> 6 heads per wave), batch 2: 4 side by side halved to 2
    assert ws_size(query_heads=24, kv_heads=4, **L) == 1024 * 2 * 2 * 6 * (128 + 2) * 4 + 1024 * 32
    # batch 8 of 4 KV heads: 8 bands of 4 streams (fewer than 32) -> 16 bands of 2
    assert ws_size(query_heads=24, kv_heads=4, batch=8, **L) == 1024 * 2 * 2 * 6 * (128 + 2) * 4 + 1024 * 32
    # batch 16 of 4 KV heads: 16 bands of 4 streams -> 2 side by side (32 bands would not be
    # halved again); batch 32: 32 bands of 4, kept
    assert ws_size(query_heads=24, kv_heads=4, batch=32, **L) == 1024 * 2 * 4 * 6 * (128 + 2) * 4 + 1024 * 32


def test_short_contexts_need_no_workspace():
    # Each sequence is one partition of the fixed route -- no merge, no workspace -- when
    # every band is short (at most 24 stream tiles), or when the longest sequence needs at
    # most 8 tiles per wave (8 waves per workgroup up to 256 workgroups, else 4) over at
    # least 64 workgroups (batch x KV heads x head chunks; here 2 KV heads, one chunk).
    assert ws_size() == 0                                                        # 8 tiles x 1
    assert ws_size(max_pages_per_sequence=24, num_physical_pages=64) == 0     # 24 tiles x 1
    assert ws_size(max_pages_per_sequence=25, num_physical_pages=64) > 0      # 25, 4 workgroups
    assert ws_size(max_context_length=384, max_pages_per_sequence=64, num_physical_pages=256) == 0
    # 32 sequences (64 workgroups of 8 waves): 64 tiles fit, 65 do not
    assert ws_size(batch=32, max_pages_per_sequence=64, num_physical_pages=4096) == 0
    assert ws_size(batch=32, max_pages_per_sequence=65, num_physical_pages=4096) > 0
    # 256 sequences (512 workgroups of 4 waves): 32 tiles fit, 33 do not
    assert ws_size(batch=256, max_pages_per_sequence=32, num_physical_pages=16384) == 0
    assert ws_size(batch=256, max_pages_per_sequence=33, num_physical_pages=16384) > 0
    # 16 sequences: 32 workgroups are too few for the per-wave rule
    assert ws_size(batch=16, max_pages_per_sequence=32, num_physical_pages=1024) > 0
    # any batch size of short sequences (2048): still one partition per sequence
    assert ws_size(batch=2048, num_physical_pages=20000) == 0
    # a route flag or a partition size keeps the caller's choice
    assert ws_size(flags=pa.PA_FLAG_FORCE_SPLIT) > 0
    # the debug bitmap still needs its words
    assert ws_size(flags=pa.PA_FLAG_DEBUG_BOUNDS) == 256


def test_workspace_size_with_partition_size():
    # a partition size may run either route (the balanced one when its partials fit it):
    # the larger of the two layouts.  Fixed partitions of one page -> 8 partitions of
    # (D + 2) floats per (sequence, head); the balanced layout with one stream side by side
    # (a partition size never takes the one-partition-per-sequence shortcut).
    bal = 1024 * 2 * 1 * 4 * (128 + 2) * 4 + 1024 * 32
    assert ws_size(partition_size=16) == max(2 * 8 * 8 * (128 + 2) * 4, bal)
    assert ws_size(partition_size=16, max_context_length=40) == max(2 * 8 * 3 * (128 + 2) * 4, bal)
    assert ws_size(partition_size=1024) == bal
    # the route flags take fixed partitions only: 128 tokens fit one partition of 1024, no
    # workspace unless split is forced
    assert ws_size(flags=pa.PA_FLAG_FORCE_SPLIT) == 2 * 8 * 1 * (128 + 2) * 4
    # PA_FLAG_FIXED_PARTITIONS keeps a partition size on the fixed route: its layout only
    assert ws_size(partition_size=16, flags=pa.PA_FLAG_FIXED_PARTITIONS) == 2 * 8 * 8 * (128 + 2) * 4
    assert ws_size(partition_size=1024, flags=pa.PA_FLAG_FIXED_PARTITIONS) == 0
    assert ws_size(flags=pa.PA_FLAG_FORCE_SINGLE, max_pages_per_sequence=64) == 0


def test_workspace_size_single_launch():
    # PA_FLAG_SINGLE_LAUNCH adds three arrival counters per workgroup slot at the end
    L = dict(max_pages_per_sequence=64, num_physical_pages=256)
    SL = pa.PA_FLAG_SINGLE_LAUNCH
    assert ws_size(flags=SL, **L) == ws_size(**L) + 1024 * 3 * 4
    assert ws_size(flags=SL | pa.PA_FLAG_DEBUG_BOUNDS, **L) == 256 + ws_size(**L) + 1024 * 3 * 4
    # short contexts are one kernel with no workspace anyway (one partition per sequence)
    assert ws_size(flags=SL) == 0


def test_workspace_size_with_bounds_bitmap():
    # PA_FLAG_DEBUG_BOUNDS puts a bitmap of batch * max_pages bits first, rounded up to 256
    # bytes; it keeps the balanced route and needs a workspace even without a merge
    D = pa.PA_FLAG_DEBUG_BOUNDS
    assert ws_size(flags=D) == 256 + ws_size()
    assert ws_size(flags=D | pa.PA_FLAG_FORCE_SINGLE) == 256
    assert ws_size(flags=D, batch=100, max_pages_per_sequence=100,
                   num_physical_pages=20000) == 1280 + ws_size(batch=100, max_pages_per_sequence=100,
                                                               num_physical_pages=20000)
    assert ws_size(flags=D | pa.PA_FLAG_FORCE_SPLIT) == 256 + ws_size(flags=pa.PA_FLAG_FORCE_SPLIT)


def test_decode_rejects_before_any_hip_call(lib):
    h = pa.pa_create(good(partition_size=16))
    need = pa.pa_workspace_size(h)
    A = 0x10000          # aligned fake device addresses: never dereferenced on these paths
    try:
        ok = dict(query=A, key_cache=A, value_cache=A, block_tables=A, context_lengths=A,
                  scale=0.1, out=A, workspace=A, workspace_bytes=need, stream=0)

        def status(**over):
            a = dict(ok)
            a.update(over)
            return lib.pa_decode(h, a["query"], a["key_cache"], a["value_cache"],
                                 a["block_tables"], a["context_lengths"], a["scale"], a["out"],
                                 a["workspace"], a["workspace_bytes"], a["stream"])
        for name in ("query", "key_cache", "value_cache", "block_tables", "context_lengths", "out"):
            assert status(**{name: None}) == pa.PA_ERR_INVALID_ARGUMENT, name
        for name in ("query", "key_cache", "value_cache", "out"):
            assert status(**{name: A + 8}) == pa.PA_ERR_MISALIGNED, name
        assert status(scale=float("nan")) == pa.PA_ERR_INVALID_ARGUMENT
        assert status(scale=float("inf")) == pa.PA_ERR_INVALID_ARGUMENT
        assert status(workspace=None) == pa.PA_ERR_WORKSPACE
        assert status(workspace_bytes=need - 1) == pa.PA_ERR_WORKSPACE
        assert status(workspace=A + 4) == pa.PA_ERR_MISALIGNED
        assert lib.pa_decode(None, A, A, A, A, A, 0.1, A, A, need, None) == pa.PA_ERR_INVALID_ARGUMENT
    finally:
        pa.pa_destroy(h)


def test_decode_noalloc_rejects_before_any_hip_call(lib):
    """pa_decode_noalloc checks what pa_decode checks, and refuses a fixed-partition problem
    whose workspace passes the library's scratch array before touching the device (the
    balanced route's size depends on the device's compute units, so its check needs one)."""
    big = pa.pa_create(good(batch=64, query_heads=32, kv_heads=8, max_pages_per_sequence=128,
                            num_physical_pages=8192, partition_size=16))
    small = pa.pa_create(good(partition_size=16))
    A = 0x10000          # aligned fake device addresses: never dereferenced on these paths
    try:
        assert pa.pa_workspace_size(big) > pa.PA_NOALLOC_SCRATCH_BYTES
        assert lib.pa_decode_noalloc(big, A, A, A, A, A, 0.1, A, None) == pa.PA_ERR_SCRATCH
        names = ("query", "key_cache", "value_cache", "block_tables", "context_lengths", "out")

        def status(scale=0.1, **over):
            a = dict.fromkeys(names, A)
            a.update(over)
            return lib.pa_decode_noalloc(small, a["query"], a["key_cache"], a["value_cache"],
                                         a["block_tables"], a["context_lengths"], scale,
                                         a["out"], None)
        for name in names:
            assert status(**{name: None}) == pa.PA_ERR_INVALID_ARGUMENT, name
        for name in ("query", "key_cache", "value_cache", "out"):
            assert status(**{name: A + 8}) == pa.PA_ERR_MISALIGNED, name
        assert status(scale=float("nan")) == pa.PA_ERR_INVALID_ARGUMENT
        assert status(scale=float("-inf")) == pa.PA_ERR_INVALID_ARGUMENT
        assert lib.pa_decode_noalloc(None, A, A, A, A, A, 0.1, A, None) == pa.PA_ERR_INVALID_ARGUMENT
        dbg = pa.pa_create(good(flags=pa.PA_FLAG_DEBUG_BOUNDS))
        try:   # the bad-entry bitmap needs a workspace the caller can read
            assert lib.pa_decode_noalloc(dbg, A, A, A, A, A, 0.1, A, None) == pa.PA_ERR_INVALID_ARGUMENT
        finally:
            pa.pa_destroy(dbg)
    finally:
        pa.pa_destroy(big)
        pa.pa_destroy(small)


def test_append_rejects_before_any_hip_call(lib):
    h = pa.pa_create(good())
    A = 0x10000          # aligned fake device addresses: never dereferenced on these paths
    try:
        names = ("new_key", "new_value", "key_cache", "value_cache", "block_tables", "positions")

        def status(**over):
            a = dict.fromkeys(names, A)
            a.update(over)
            return lib.pa_append(h, *(a[n] for n in names), None)
        for name in names:
            assert status(**{name: None}) == pa.PA_ERR_INVALID_ARGUMENT, name
        for name in ("new_key", "new_value", "key_cache", "value_cache"):
            assert status(**{name: A + 8}) == pa.PA_ERR_MISALIGNED, name
        assert lib.pa_append(None, A, A, A, A, A, A, None) == pa.PA_ERR_INVALID_ARGUMENT
    finally:
        pa.pa_destroy(h)


def test_status_strings(lib):
    names = ["PA_OK", "PA_ERR_INVALID_ARGUMENT", "PA_ERR_UNSUPPORTED", "PA_ERR_MISALIGNED",
             "PA_ERR_WORKSPACE", "PA_ERR_HIP", "PA_ERR_NO_MEMORY", "PA_ERR_SCRATCH"]
    for i, n in enumerate(names):
        assert pa.pa_status_string(i) == n
    assert pa.pa_status_string(99) == "PA_ERR_UNKNOWN"


def test_binding_does_not_route_through_the_oracle():
    """The product package never imports the oracle and has no CPU fallback."""
    pkg = os.path.join(ROOT, "decode_attention_paged_03_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", text, re.M), f
                assert "pa_oracle" not in text and "libpa_oracle" not in text, f
