"""ctypes front end of the fp64 CPU oracle (oracle/pa_oracle.c).

TEST INFRASTRUCTURE ONLY: only the tests, the smoke check and the benchmark's
CPU-baseline leg use it.  Arguments are numpy arrays: fp16 query / key / value
(any array whose bytes are IEEE binary16), int32 block tables and context lengths.
The arithmetic lives entirely in pa_oracle.c.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libpa_oracle.so")
_libs = {}

_ERRORS = {1: "bad argument", 2: "context length or block-table entry outside the pool",
           3: "out of host memory"}


def _load(path: Optional[str] = None):
    """Load the oracle library (default: oracle/libpa_oracle.so, built on first use)."""
    path = path or _LIB_PATH
    if path in _libs:
        return _libs[path]
    if path == _LIB_PATH and not os.path.exists(path):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I = ctypes.c_int
    lib.pa_oracle_half_to_double.argtypes = [ctypes.c_uint16]
    lib.pa_oracle_half_to_double.restype = ctypes.c_double
    common = [I, I, I, I, I, I, I, P, P, P, P, P, ctypes.c_double]
    lib.pa_oracle_attend.argtypes = common + [P, I, I, P]
    lib.pa_oracle_attend.restype = I
    lib.pa_oracle_attend_zero_pages.argtypes = common + [P, I, I, P]
    lib.pa_oracle_attend_zero_pages.restype = I
    lib.pa_oracle_bad_entries.argtypes = [I, I, I, I, P, P, P]
    lib.pa_oracle_bad_entries.restype = ctypes.c_longlong
    lib.pa_oracle_attend_partitioned.argtypes = common + [I, P, I, I, P]
    lib.pa_oracle_attend_partitioned.restype = I
    lib.pa_oracle_append.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, P]
    lib.pa_oracle_append.restype = I
    lib.pa_oracle_max_threads.argtypes = []
    lib.pa_oracle_max_threads.restype = I
    _libs[path] = lib
    return lib


def half_to_double(bits: int, lib_path: Optional[str] = None) -> float:
    return _load(lib_path).pa_oracle_half_to_double(int(bits) & 0xFFFF)


def max_threads() -> int:
    return _load().pa_oracle_max_threads()


def _prep(query, key_cache, value_cache, block_tables, context_lengths):
    q = np.ascontiguousarray(query).view(np.uint16)
    k = np.ascontiguousarray(key_cache).view(np.uint16)
    v = np.ascontiguousarray(value_cache).view(np.uint16)
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    ctx = np.ascontiguousarray(context_lengths, dtype=np.int32)
    if q.ndim != 3 or k.ndim != 4 or v.shape != k.shape or bt.ndim != 2:
        raise ValueError("expected q [B][QH][D], K/V [pages][page_size][KVH][D], bt [B][max_pages]")
    B, QH, D = q.shape
    num_pages, ps, KVH, D2 = k.shape
    if D2 != D or bt.shape[0] != B or ctx.shape != (B,):
        raise ValueError("inconsistent shapes")
    return q, k, v, bt, ctx, (B, QH, KVH, D, ps, bt.shape[1], num_pages)


def _call(fn_name, query, key_cache, value_cache, block_tables, context_lengths, scale,
          rows, nthreads, extra=(), lib_path=None):
    lib = _load(lib_path)
    q, k, v, bt, ctx, dims = _prep(query, key_cache, value_cache, block_tables, context_lengths)
    B, QH, KVH, D = dims[0], dims[1], dims[2], dims[3]
    if rows is None:
        out = np.zeros((B, QH, D), dtype=np.float64)
        rows_arr, n_rows, rows_ptr = None, 0, None
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int32).reshape(-1))
        n_rows = int(rows_arr.size)
        out = np.zeros((n_rows, D), dtype=np.float64)
        rows_ptr = rows_arr.ctypes.data
    rc = getattr(lib, fn_name)(*dims, q.ctypes.data, k.ctypes.data, v.ctypes.data,
                               bt.ctypes.data, ctx.ctypes.data, float(scale), *extra,
                               rows_ptr, n_rows, int(nthreads), out.ctypes.data)
    if rc:
        raise ValueError(f"oracle: {_ERRORS.get(rc, rc)}")
    return out


def attend(query, key_cache, value_cache, block_tables, context_lengths, scale: float,
           rows: Optional[Sequence[int]] = None, nthreads: int = 1,
           lib_path: Optional[str] = None, zero_pages: bool = False) -> np.ndarray:
    """Direct definition in fp64.  ``rows``: flat b*query_heads+h indices to evaluate
    (returns [len(rows)][D]); default all (returns [B][QH][D]).  ``lib_path`` selects
    another build of pa_oracle.c (the tests use it for deliberately broken copies).
    ``zero_pages``: table entries outside the pool read as pages of zero keys and values
    (the debug-bounds reading) instead of being an error."""
    return _call("pa_oracle_attend_zero_pages" if zero_pages else "pa_oracle_attend", query,
                 key_cache, value_cache, block_tables, context_lengths, scale, rows, nthreads,
                 lib_path=lib_path)


def bad_entries(block_tables, context_lengths, page_size: int, num_pages: int,
                lib_path: Optional[str] = None):
    """(bitmap, count): the dereferenced table entries outside the pool, as uint32 words
    (bit b * max_pages + lp), and how many there are."""
    lib = _load(lib_path)
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    ctx = np.ascontiguousarray(context_lengths, dtype=np.int32)
    B, max_pages = bt.shape
    bitmap = np.zeros((B * max_pages + 31) // 32, dtype=np.uint32)
    n = lib.pa_oracle_bad_entries(B, int(page_size), max_pages, int(num_pages), bt.ctypes.data,
                                  ctx.ctypes.data, bitmap.ctypes.data)
    if n < 0:
        raise ValueError("oracle: bad argument")
    return bitmap, int(n)


def attend_partitioned(query, key_cache, value_cache, block_tables, context_lengths,
                       scale: float, partition_size: int,
                       rows: Optional[Sequence[int]] = None, nthreads: int = 1,
                       lib_path: Optional[str] = None) -> np.ndarray:
    """The same result through per-partition (max, sum, acc) triples and their combination."""
    return _call("pa_oracle_attend_partitioned", query, key_cache, value_cache, block_tables,
                 context_lengths, scale, rows, nthreads, extra=(int(partition_size),),
                 lib_path=lib_path)


def attend_workload(wl, rows=None, nthreads: int = 1, partition_size: int = 0) -> np.ndarray:
    """Convenience: evaluate a ``workloads.Workload``-shaped object."""
    if partition_size:
        return attend_partitioned(wl.query, wl.key_cache, wl.value_cache, wl.block_tables,
                                  wl.context_lengths, wl.scale, partition_size, rows, nthreads)
    return attend(wl.query, wl.key_cache, wl.value_cache, wl.block_tables, wl.context_lengths,
                  wl.scale, rows, nthreads)


def append(new_key, new_value, block_tables, positions, key_cache, value_cache,
           lib_path: Optional[str] = None):
    """Store one new token per sequence: returns (key_cache', value_cache', n_written),
    copies of the caches with new_key[b] / new_value[b] ([batch][kv_heads][head_dim] fp16)
    written at position positions[b] of sequence b (skipped when negative or when the
    position names no slot of the pool).  The input caches are left untouched."""
    lib = _load(lib_path)
    k = np.array(key_cache, copy=True, order="C").view(np.uint16)
    v = np.array(value_cache, copy=True, order="C").view(np.uint16)
    nk = np.ascontiguousarray(new_key).view(np.uint16)
    nv = np.ascontiguousarray(new_value).view(np.uint16)
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    pos = np.ascontiguousarray(positions, dtype=np.int32)
    if k.ndim != 4 or v.shape != k.shape or bt.ndim != 2:
        raise ValueError("expected K/V [pages][page_size][KVH][D] and bt [B][max_pages]")
    num_pages, ps, KVH, D = k.shape
    B = bt.shape[0]
    if nk.shape != (B, KVH, D) or nv.shape != nk.shape or pos.shape != (B,):
        raise ValueError("inconsistent shapes")
    n = ctypes.c_int(0)
    rc = lib.pa_oracle_append(B, KVH, D, ps, bt.shape[1], num_pages, nk.ctypes.data,
                              nv.ctypes.data, bt.ctypes.data, pos.ctypes.data, k.ctypes.data,
                              v.ctypes.data, ctypes.addressof(n))
    if rc:
        raise ValueError(f"oracle: {_ERRORS.get(rc, rc)}")
    return k.view(np.float16), v.view(np.float16), int(n.value)
