"""MI355X-native paged grouped-query attention: KV append with RoPE, split-context
decode and chunked prefill over a shared pool of 16-token pages.

The compute lives in ``libpa.so`` (hand-written HIP kernels for gfx950 behind a
C ABI, declared in ``include/pa.h``).  :mod:`.binding` is a thin ctypes layer
over it that takes torch device tensors; it raises if the library has not been
built, it never falls back to another implementation.
"""
from .workloads import HEAD_DIM, NUM_KV_HEADS, NUM_Q_HEADS, PAGE_SIZE, ROPE_THETA  # noqa: F401

__all__ = ["HEAD_DIM", "NUM_KV_HEADS", "NUM_Q_HEADS", "PAGE_SIZE", "ROPE_THETA"]
