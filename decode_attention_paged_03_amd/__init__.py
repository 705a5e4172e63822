"""MI355X (gfx950) paged-attention decode engine.

The compute path is a C-ABI HIP library (``libpa.so``, built from ``csrc/``);
``decode_attention_paged_03_amd.pa`` is its thin ctypes binding.  Importing the
package does not load the library; ``pa.load()`` does, and raises if it is missing.
"""
__all__ = ["pa", "workloads"]
