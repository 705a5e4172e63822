"""ctypes binding of libpa.so -- argument marshalling only.

The functions below carry the C ABI's names (``pa_create``, ``pa_workspace_size``,
``pa_decode``, ``pa_decode_noalloc``, ``pa_append``, ``pa_destroy``, ``pa_status_string``) and
take plain integers for device pointers and the stream.  ``PagedDecoder`` is a
convenience wrapper that takes torch tensors, checks their dtype / device / contiguity
and passes their ``data_ptr()`` through; every step of the computation runs in the library's HIP
kernels.  There is no fallback: if ``libpa.so`` is missing, ``load()`` raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpa.so")

PA_OK = 0
PA_ERR_INVALID_ARGUMENT = 1
PA_ERR_UNSUPPORTED = 2
PA_ERR_MISALIGNED = 3
PA_ERR_WORKSPACE = 4
PA_ERR_HIP = 5
PA_ERR_NO_MEMORY = 6
PA_ERR_SCRATCH = 7

PA_NOALLOC_SCRATCH_BYTES = 32 << 20

PA_FLAG_FORCE_SPLIT = 0x1
PA_FLAG_FORCE_SINGLE = 0x2
PA_FLAG_DEBUG_BOUNDS = 0x4
PA_FLAG_SINGLE_LAUNCH = 0x8
PA_FLAG_FIXED_PARTITIONS = 0x10

EXPORTED = ("pa_create", "pa_workspace_size", "pa_decode", "pa_decode_noalloc", "pa_append",
            "pa_destroy", "pa_status_string")


class pa_problem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("query_heads", ctypes.c_int32),
                ("kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("max_pages_per_sequence", ctypes.c_int32),
                ("num_physical_pages", ctypes.c_int32), ("partition_size", ctypes.c_int32),
                ("max_context_length", ctypes.c_int32), ("flags", ctypes.c_uint32)]


class PaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {pa_status_string(status)} ({status})")


_lib = None


def load() -> ctypes.CDLL:
    """Load libpa.so (built in-tree by ``decode_attention_paged_03_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m decode_attention_paged_03_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    lib.pa_create.argtypes = [ctypes.POINTER(pa_problem), ctypes.POINTER(ctypes.c_void_p)]
    lib.pa_create.restype = ctypes.c_int
    lib.pa_workspace_size.argtypes = [P, ctypes.POINTER(ctypes.c_size_t)]
    lib.pa_workspace_size.restype = ctypes.c_int
    lib.pa_decode.argtypes = [P, P, P, P, P, P, ctypes.c_float, P, P, ctypes.c_size_t, P]
    lib.pa_decode.restype = ctypes.c_int
    lib.pa_decode_noalloc.argtypes = [P, P, P, P, P, P, ctypes.c_float, P, P]
    lib.pa_decode_noalloc.restype = ctypes.c_int
    lib.pa_append.argtypes = [P, P, P, P, P, P, P, P]
    lib.pa_append.restype = ctypes.c_int
    lib.pa_destroy.argtypes = [P]
    lib.pa_destroy.restype = ctypes.c_int
    lib.pa_status_string.argtypes = [ctypes.c_int]
    lib.pa_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def pa_status_string(status: int) -> str:
    return load().pa_status_string(int(status)).decode()


def pa_create(problem: pa_problem) -> ctypes.c_void_p:
    h = ctypes.c_void_p()
    st = load().pa_create(ctypes.byref(problem), ctypes.byref(h))
    if st != PA_OK:
        raise PaError(st, "pa_create")
    return h


def pa_workspace_size(handle) -> int:
    n = ctypes.c_size_t()
    st = load().pa_workspace_size(handle, ctypes.byref(n))
    if st != PA_OK:
        raise PaError(st, "pa_workspace_size")
    return int(n.value)


def pa_decode(handle, query: int, key_cache: int, value_cache: int, block_tables: int,
              context_lengths: int, scale: float, out: int, workspace: int,
              workspace_bytes: int, stream: int) -> None:
    st = load().pa_decode(handle, query, key_cache, value_cache, block_tables, context_lengths,
                          float(scale), out, workspace or None, int(workspace_bytes), stream or None)
    if st != PA_OK:
        raise PaError(st, "pa_decode")


def pa_decode_noalloc(handle, query: int, key_cache: int, value_cache: int, block_tables: int,
                      context_lengths: int, scale: float, out: int, stream: int) -> None:
    st = load().pa_decode_noalloc(handle, query, key_cache, value_cache, block_tables,
                                  context_lengths, float(scale), out, stream or None)
    if st != PA_OK:
        raise PaError(st, "pa_decode_noalloc")


def pa_append(handle, new_key: int, new_value: int, key_cache: int, value_cache: int,
              block_tables: int, positions: int, stream: int) -> None:
    st = load().pa_append(handle, new_key, new_value, key_cache, value_cache, block_tables,
                          positions, stream or None)
    if st != PA_OK:
        raise PaError(st, "pa_append")


def pa_destroy(handle) -> None:
    st = load().pa_destroy(handle)
    if st != PA_OK:
        raise PaError(st, "pa_destroy")


def make_problem(*, batch, query_heads, kv_heads, head_dim, page_size, max_pages_per_sequence,
                 num_physical_pages, partition_size=0, max_context_length=0, flags=0) -> pa_problem:
    return pa_problem(batch, query_heads, kv_heads, head_dim, page_size, max_pages_per_sequence,
                      num_physical_pages, partition_size, max_context_length, flags)


class PagedDecoder:
    """A handle plus a workspace, called with torch tensors on one GPU."""

    def __init__(self, problem: pa_problem, device="cuda"):
        import torch
        self.problem = problem
        self.handle = pa_create(problem)
        self.workspace_bytes = pa_workspace_size(self.handle)
        # PA_FLAG_SINGLE_LAUNCH keeps arrival counters in the workspace, zero before the first
        # call (every call leaves them at zero)
        alloc = torch.zeros if problem.flags & PA_FLAG_SINGLE_LAUNCH else torch.empty
        self.workspace = (alloc(self.workspace_bytes, dtype=torch.uint8, device=device)
                          if self.workspace_bytes else None)

    def __call__(self, query, key_cache, value_cache, block_tables, context_lengths, scale,
                 out=None, stream=None):
        out, stream = self._check(query, key_cache, value_cache, block_tables, context_lengths,
                                  out, stream)
        ws = self.workspace
        pa_decode(self.handle, query.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(),
                  block_tables.data_ptr(), context_lengths.data_ptr(), scale, out.data_ptr(),
                  ws.data_ptr() if ws is not None else 0, self.workspace_bytes, stream.cuda_stream)
        return out

    def bind(self, query, key_cache, value_cache, block_tables, context_lengths, scale, out,
             stream=None):
        """The same call with its arguments checked and converted once: returns a function
        of no arguments that enqueues pa_decode on these buffers (whose contents may change
        between calls), for loops that repeat one decode step.  It keeps the tensors alive;
        calling it after close() raises."""
        out, stream = self._check(query, key_cache, value_cache, block_tables, context_lengths,
                                  out, stream)
        ws = self.workspace
        P = ctypes.c_void_p
        fn = load().pa_decode
        args = (self.handle, P(query.data_ptr()), P(key_cache.data_ptr()), P(value_cache.data_ptr()),
                P(block_tables.data_ptr()), P(context_lengths.data_ptr()), ctypes.c_float(scale),
                P(out.data_ptr()), P(ws.data_ptr() if ws is not None else None),
                ctypes.c_size_t(self.workspace_bytes), P(stream.cuda_stream))
        keep = (query, key_cache, value_cache, block_tables, context_lengths, out, ws, stream)

        def call():
            if self.handle is None:
                raise ValueError("the decoder was closed")
            st = fn(*args)
            if st != PA_OK:
                raise PaError(st, "pa_decode")
            return keep[5]
        return call

    def _check(self, query, key_cache, value_cache, block_tables, context_lengths, out, stream):
        import torch
        p = self.problem
        for name, t, dt in (("query", query, torch.float16), ("key_cache", key_cache, torch.float16),
                            ("value_cache", value_cache, torch.float16),
                            ("block_tables", block_tables, torch.int32),
                            ("context_lengths", context_lengths, torch.int32)):
            if t.dtype != dt or not t.is_cuda or not t.is_contiguous():
                raise ValueError(f"{name}: need a contiguous {dt} CUDA tensor")
        if tuple(query.shape) != (p.batch, p.query_heads, p.head_dim):
            raise ValueError("query shape")
        if tuple(key_cache.shape[1:]) != (p.page_size, p.kv_heads, p.head_dim) or \
                key_cache.shape != value_cache.shape:
            raise ValueError("key/value cache shape")
        if tuple(block_tables.shape) != (p.batch, p.max_pages_per_sequence):
            raise ValueError("block table shape")
        if tuple(context_lengths.shape) != (p.batch,):
            raise ValueError("context length shape")
        if out is None:
            out = torch.empty((p.batch, p.query_heads, p.head_dim), dtype=torch.float32,
                              device=query.device)
        elif out.dtype != torch.float32 or not out.is_contiguous() or \
                tuple(out.shape) != (p.batch, p.query_heads, p.head_dim):
            raise ValueError("out: need a contiguous float32 [batch][query_heads][head_dim] tensor")
        if stream is None:
            stream = torch.cuda.current_stream(query.device)
        return out, stream

    def bad_entry_bitmap(self):
        """With PA_FLAG_DEBUG_BOUNDS: the bitmap the last call left at the start of the
        workspace, as numpy uint32 words (bit i of word w: table entry 32 w + i, row-major),
        copied to the host after the device has finished."""
        import numpy as np
        import torch
        p = self.problem
        if not (p.flags & PA_FLAG_DEBUG_BOUNDS):
            raise ValueError("the problem was created without PA_FLAG_DEBUG_BOUNDS")
        words = (p.batch * p.max_pages_per_sequence + 31) // 32
        torch.cuda.synchronize(self.workspace.device)
        return self.workspace[:4 * words].cpu().numpy().view(np.uint32).copy()

    def append(self, new_key, new_value, key_cache, value_cache, block_tables, positions,
               stream=None):
        """Store new_key[b] / new_value[b] ([batch][kv_heads][head_dim] fp16) at position
        positions[b] of sequence b, in place in key_cache / value_cache."""
        import torch
        p = self.problem
        for name, t, dt in (("new_key", new_key, torch.float16),
                            ("new_value", new_value, torch.float16),
                            ("key_cache", key_cache, torch.float16),
                            ("value_cache", value_cache, torch.float16),
                            ("block_tables", block_tables, torch.int32),
                            ("positions", positions, torch.int32)):
            if t.dtype != dt or not t.is_cuda or not t.is_contiguous():
                raise ValueError(f"{name}: need a contiguous {dt} CUDA tensor")
        if tuple(new_key.shape) != (p.batch, p.kv_heads, p.head_dim) or \
                new_value.shape != new_key.shape:
            raise ValueError("new key/value shape")
        if tuple(key_cache.shape) != (p.num_physical_pages, p.page_size, p.kv_heads, p.head_dim) \
                or key_cache.shape != value_cache.shape:
            raise ValueError("key/value cache shape")
        if tuple(block_tables.shape) != (p.batch, p.max_pages_per_sequence):
            raise ValueError("block table shape")
        if tuple(positions.shape) != (p.batch,):
            raise ValueError("positions shape")
        if stream is None:
            stream = torch.cuda.current_stream(new_key.device)
        pa_append(self.handle, new_key.data_ptr(), new_value.data_ptr(), key_cache.data_ptr(),
                  value_cache.data_ptr(), block_tables.data_ptr(), positions.data_ptr(),
                  stream.cuda_stream)

    def close(self):
        if self.handle:
            pa_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def decoder_for(wl, *, partition_size: Optional[int] = None, flags: int = 0,
                max_context_length: int = 0, device="cuda") -> PagedDecoder:
    """A decoder sized for a ``workloads.Workload``."""
    prob = make_problem(batch=wl.batch, query_heads=wl.query_heads, kv_heads=wl.kv_heads,
                        head_dim=wl.head_dim, page_size=wl.page_size,
                        max_pages_per_sequence=wl.max_pages_per_sequence,
                        num_physical_pages=wl.num_pages,
                        partition_size=wl.partition_size if partition_size is None else partition_size,
                        max_context_length=max_context_length, flags=flags)
    return PagedDecoder(prob, device=device)
