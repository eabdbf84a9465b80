"""ctypes binding of libpa.so (include/pa.h) for torch device tensors.

Argument marshalling only: shapes, dtypes and devices are checked, raw device
pointers and torch's current HIP stream are handed to the C ABI, and a non-zero
status becomes a :class:`PaError`.  All work runs in the library's HIP kernels;
if ``libpa.so`` is missing this module raises instead of computing anything
another way.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np
import torch

from . import workloads as _w

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpa.so")
_lib = None

PA_OK, PA_ERR_INVALID_ARG, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE, PA_ERR_HIP, PA_ERR_REJECTED = range(6)
PA_BATCH_CONTINUOUS, PA_BATCH_STATIC = 0, 1
PA_OUT_BF16, PA_OUT_FP32 = 0, 1
PA_DEVERR_CONTEXT_LEN, PA_DEVERR_PAGE_ID, PA_DEVERR_DISPATCH_ORDER = 0x1, 0x2, 0x4

EXPORTS = ("pa_status_string", "pa_abi_version", "pa_rope_table_fill_host", "pa_append_kv_rope",
           "pa_decode_workspace_bytes", "pa_decode_partition_tokens", "pa_decode_gqa", "pa_append_decode_gqa",
           "pa_prefill_chunk", "pa_admission_credit_pages", "pa_kvm_create", "pa_kvm_destroy", "pa_kvm_submit",
           "pa_kvm_schedule", "pa_kvm_set_length", "pa_kvm_release", "pa_kvm_block_tables", "pa_kvm_lengths",
           "pa_kvm_slot_request", "pa_kvm_slot_budget", "pa_kvm_free_pages", "pa_kvm_reserved_pages",
           "pa_kvm_queued", "pa_i8_pool_bytes", "pa_quantize_pages_i8", "pa_append_kv_rope_i8", "pa_decode_gqa_i8",
           "pa_append_decode_gqa_i8", "pa_argmax_workspace_bytes", "pa_argmax", "pa_probe_stream_read",
           "pa_dispatch_order_longest_first", "pa_get_device_error", "pa_build_id",
           "pa_append_decode_gqa_noalloc", "pa_order_by_length", "pa_prefill_chunk_i8")
PA_LOGITS_BF16, PA_LOGITS_FP32 = 0, 1
PA_I8_TILE_BYTES = 2176
# PA_ABI_VERSION of the header whose signatures this module declares
ABI_VERSION = 14


class PaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


def _require_abi(found: int) -> None:
    """A library built from another header would be called with the wrong argument lists."""
    if found != ABI_VERSION:
        raise RuntimeError(f"{_LIB_PATH} has ABI version {found}, this binding expects {ABI_VERSION}: "
                           "rebuild it with paged_kv_gqa_append_amd.build.build()")


def _require_current(built_id: str) -> None:
    """A library built from older sources than the ones beside it would run stale kernels."""
    from . import build as _build

    want = _build.source_digest()
    if built_id != want:
        raise RuntimeError(f"{_LIB_PATH} was built from other sources (build id {built_id[:12]}..., the tree's "
                           f"sources hash to {want[:12]}...): rebuild it with "
                           "paged_kv_gqa_append_amd.build.build()")


def lib():
    """Load libpa.so (raises if it has not been built, was built from another header, or from
    sources other than the ones in the tree)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it with paged_kv_gqa_append_amd.build.build() "
                           "(there is no fallback implementation)")
    L = ctypes.CDLL(_LIB_PATH)
    L.pa_abi_version.restype = ctypes.c_int32
    L.pa_abi_version.argtypes = []
    _require_abi(int(L.pa_abi_version()))
    L.pa_build_id.restype = ctypes.c_char_p
    L.pa_build_id.argtypes = []
    _require_current(L.pa_build_id().decode())
    P, i32, u64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    L.pa_status_string.restype = ctypes.c_char_p
    L.pa_status_string.argtypes = [ctypes.c_int]
    L.pa_abi_version.restype = i32
    L.pa_abi_version.argtypes = []
    L.pa_rope_table_fill_host.restype = ctypes.c_int
    L.pa_rope_table_fill_host.argtypes = [P, i32, ctypes.c_double]
    L.pa_append_kv_rope.restype = ctypes.c_int
    L.pa_append_kv_rope.argtypes = [P, P, P, P, P, P, P, P, i32, i32, i32, i32, i32, P, P]
    L.pa_decode_workspace_bytes.restype = u64
    L.pa_decode_workspace_bytes.argtypes = [i32, i32]
    L.pa_decode_partition_tokens.restype = i32
    L.pa_decode_partition_tokens.argtypes = []
    L.pa_decode_gqa.restype = ctypes.c_int
    L.pa_decode_gqa.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, ctypes.c_float, i32, P, u64, P, P, P, P]
    L.pa_append_decode_gqa.restype = ctypes.c_int
    L.pa_append_decode_gqa.argtypes = [P, P, P, P, P, P, P, P, P, i32, i32, i32, i32, i32, ctypes.c_float, i32, P,
                                       u64, P, P, P, P]
    L.pa_append_decode_gqa_noalloc.restype = ctypes.c_int
    L.pa_append_decode_gqa_noalloc.argtypes = [P, P, P, P, P, P, P, P, P, i32, i32, i32, i32, i32, ctypes.c_float,
                                               i32, P, P, P, P]
    L.pa_prefill_chunk.restype = ctypes.c_int
    L.pa_prefill_chunk.argtypes = [P, P, P, P, P, P, P, P, P, i32, i32, i32, i32, i32, i32, ctypes.c_float, i32,
                                   P, P]
    L.pa_prefill_chunk_i8.restype = ctypes.c_int
    L.pa_prefill_chunk_i8.argtypes = [P, P, P, P, P, P, P, P, i32, i32, i32, i32, i32, i32, ctypes.c_float, i32, P,
                                      P]
    L.pa_i8_pool_bytes.restype = u64
    L.pa_i8_pool_bytes.argtypes = [i32]
    L.pa_quantize_pages_i8.restype = ctypes.c_int
    L.pa_quantize_pages_i8.argtypes = [P, P, P, P, i32, i32, P, P]
    L.pa_append_kv_rope_i8.restype = ctypes.c_int
    L.pa_append_kv_rope_i8.argtypes = [P, P, P, P, P, P, P, i32, i32, i32, i32, i32, P, P]
    L.pa_decode_gqa_i8.restype = ctypes.c_int
    L.pa_decode_gqa_i8.argtypes = [P, P, P, P, P, i32, i32, i32, i32, ctypes.c_float, i32, P, u64, P, P, P, P]
    L.pa_append_decode_gqa_i8.restype = ctypes.c_int
    L.pa_append_decode_gqa_i8.argtypes = [P, P, P, P, P, P, P, P, i32, i32, i32, i32, i32, ctypes.c_float, i32, P,
                                          u64, P, P, P, P]
    L.pa_argmax_workspace_bytes.restype = u64
    L.pa_argmax_workspace_bytes.argtypes = [i32, i32, i32]
    L.pa_argmax.restype = ctypes.c_int
    L.pa_argmax.argtypes = [P, P, i32, i32, i32, P, u64, P]
    L.pa_dispatch_order_longest_first.restype = ctypes.c_int
    L.pa_dispatch_order_longest_first.argtypes = [P, i32, P]
    L.pa_order_by_length.restype = ctypes.c_int
    L.pa_order_by_length.argtypes = [P, i32, i32, i32, i32, P, P]
    L.pa_probe_stream_read.restype = ctypes.c_int
    L.pa_probe_stream_read.argtypes = [P, u64, P, P]
    L.pa_get_device_error.restype = i32
    L.pa_get_device_error.argtypes = [P, i32, P]
    i64 = ctypes.c_int64
    L.pa_admission_credit_pages.restype = i64
    L.pa_admission_credit_pages.argtypes = [i32, i32, i32]
    L.pa_kvm_create.restype = ctypes.c_int
    L.pa_kvm_create.argtypes = [i32, i32, i32, i32, i32, ctypes.POINTER(P)]
    L.pa_kvm_destroy.restype = None
    L.pa_kvm_destroy.argtypes = [P]
    L.pa_kvm_submit.restype = ctypes.c_int
    L.pa_kvm_submit.argtypes = [P, i32, i32, ctypes.POINTER(i32)]
    L.pa_kvm_schedule.restype = i32
    L.pa_kvm_schedule.argtypes = [P, P, i32]
    L.pa_kvm_set_length.restype = ctypes.c_int
    L.pa_kvm_set_length.argtypes = [P, i32, i32]
    L.pa_kvm_release.restype = ctypes.c_int
    L.pa_kvm_release.argtypes = [P, i32]
    for name in ("pa_kvm_block_tables", "pa_kvm_lengths"):
        getattr(L, name).restype = ctypes.POINTER(i32)
        getattr(L, name).argtypes = [P]
    for name in ("pa_kvm_slot_request", "pa_kvm_slot_budget"):
        getattr(L, name).restype = i32
        getattr(L, name).argtypes = [P, i32]
    for name, rt in (("pa_kvm_free_pages", i32), ("pa_kvm_reserved_pages", i64), ("pa_kvm_queued", i32)):
        getattr(L, name).restype = rt
        getattr(L, name).argtypes = [P]
    _lib = L
    return L


def get_device_error(device_flags: torch.Tensor, clear: bool = False, stream=None) -> int:
    """pa_get_device_error: wait for the stream, return the PA_DEVERR_* bits of the caller's
    device flag word (and reset it to 0 when ``clear``).  Synchronises: a debug helper."""
    _expect(device_flags, "device_flags", torch.int32, (1,))
    rc = int(lib().pa_get_device_error(_ptr(device_flags), 1 if clear else 0, _stream(stream)))
    if rc < 0:
        raise PaError(-rc, "pa_get_device_error")
    return rc


def status_string(status: int) -> str:
    return lib().pa_status_string(int(status)).decode()


def _check(rc: int, where: str) -> None:
    if rc != PA_OK:
        raise PaError(rc, where)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _order(dispatch_order, num_seqs: int, device=None):
    """The two order arguments of a decode call, (keep-alive, host pointer, device pointer), from
    an optional dispatch order.  A torch tensor on the call's device is a device order
    (int32[num_seqs], e.g. from order_by_length), passed as device_order; anything else is a host
    order: a contiguous int32 numpy array is used as it is, other sequences are copied.  The
    library reads exactly num_seqs entries, so an order of any other length is refused here."""
    if dispatch_order is None:
        return None, None, None
    if isinstance(dispatch_order, torch.Tensor):
        _expect(dispatch_order, "dispatch_order", torch.int32, (int(num_seqs),), device)
        return dispatch_order, None, _ptr(dispatch_order)
    arr = dispatch_order
    if not (isinstance(arr, np.ndarray) and arr.dtype == np.int32 and arr.flags.c_contiguous):
        arr = np.ascontiguousarray(np.asarray(dispatch_order, dtype=np.int32))
    if arr.shape != (int(num_seqs),):
        raise ValueError(f"dispatch_order must be a 1-D array of exactly num_seqs = {int(num_seqs)} sequence "
                         f"indices, got shape {arr.shape}")
    return arr, ctypes.c_void_p(arr.ctypes.data), None


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _expect(t: torch.Tensor, name: str, dtype, shape=None, device=None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def rope_table(max_pos: int, theta: float = _w.ROPE_THETA, device="cuda") -> torch.Tensor:
    """[max_pos][32][2] fp64 (cos, sin) table, filled by the library on the host, then uploaded."""
    host = np.empty((max_pos, _w.HEAD_DIM // 2, 2), dtype=np.float64)
    _check(lib().pa_rope_table_fill_host(host.ctypes.data_as(ctypes.c_void_p), int(max_pos), float(theta)),
           "pa_rope_table_fill_host")
    return torch.from_numpy(host).to(device)


def decode_workspace_bytes(num_seqs: int, max_blocks: int) -> int:
    return int(lib().pa_decode_workspace_bytes(int(num_seqs), int(max_blocks)))


def decode_partition_tokens() -> int:
    return int(lib().pa_decode_partition_tokens())


def decode_workspace(num_seqs: int, max_blocks: int, device="cuda") -> Optional[torch.Tensor]:
    n = decode_workspace_bytes(num_seqs, max_blocks)
    return None if n == 0 else torch.empty(n // 4, dtype=torch.float32, device=device)


def _pool_checks(k_pool, v_pool):
    _expect(k_pool, "k_pool", torch.bfloat16)
    _expect(v_pool, "v_pool", torch.bfloat16, shape=k_pool.shape, device=k_pool.device)
    if k_pool.dim() != 4 or tuple(k_pool.shape[1:]) != (_w.NUM_KV_HEADS, _w.PAGE_SIZE, _w.HEAD_DIM):
        raise ValueError(f"pools must be [num_pages][8][16][64], got {tuple(k_pool.shape)}")
    return int(k_pool.shape[0])


def append_kv_rope(q: Optional[torch.Tensor], k_new: torch.Tensor, v_new: torch.Tensor, k_pool: torch.Tensor,
                   v_pool: torch.Tensor, block_tables: torch.Tensor, context_lens: torch.Tensor,
                   rope_cos_sin: torch.Tensor, device_flags: Optional[torch.Tensor] = None, page_size: int = 16,
                   stream=None) -> None:
    """pa_append_kv_rope: write RoPE(k_new), v_new at pos = L-1; rotate q in place (if given)."""
    num_pages = _pool_checks(k_pool, v_pool)
    dev = k_pool.device
    _expect(context_lens, "context_lens", torch.int32, device=dev)
    B = int(context_lens.shape[0])
    _expect(block_tables, "block_tables", torch.int32, device=dev)
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [num_seqs][max_blocks]")
    _expect(k_new, "k_new", torch.bfloat16, (B, 8, 64), dev)
    _expect(v_new, "v_new", torch.bfloat16, (B, 8, 64), dev)
    if q is not None:
        _expect(q, "q", torch.bfloat16, (B, 32, 64), dev)
    _expect(rope_cos_sin, "rope_cos_sin", torch.float64, device=dev)
    if device_flags is not None:
        _expect(device_flags, "device_flags", torch.int32, (1,), dev)
    rc = lib().pa_append_kv_rope(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables),
                                 _ptr(context_lens), _ptr(rope_cos_sin), B, int(block_tables.shape[1]), num_pages,
                                 int(page_size), int(rope_cos_sin.shape[0]), _ptr(device_flags), _stream(stream))
    _check(rc, "pa_append_kv_rope")


def decode_gqa(out: torch.Tensor, q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
               block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float = 0.125,
               workspace: Optional[torch.Tensor] = None, device_flags: Optional[torch.Tensor] = None,
               page_size: int = 16, dispatch_order=None, stream=None) -> torch.Tensor:
    """pa_decode_gqa into ``out`` ([B][32][64] bf16 or fp32; may be ``q`` itself)."""
    num_pages = _pool_checks(k_pool, v_pool)
    dev = k_pool.device
    _expect(context_lens, "context_lens", torch.int32, device=dev)
    B = int(context_lens.shape[0])
    _expect(block_tables, "block_tables", torch.int32, device=dev)
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [num_seqs][max_blocks]")
    _expect(q, "q", torch.bfloat16, (B, 32, 64), dev)
    if out.dtype == torch.bfloat16:
        odt = PA_OUT_BF16
    elif out.dtype == torch.float32:
        odt = PA_OUT_FP32
    else:
        raise TypeError("out must be bfloat16 or float32")
    _expect(out, "out", out.dtype, (B, 32, 64), dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if device_flags is not None:
        _expect(device_flags, "device_flags", torch.int32, (1,), dev)
    order_keep, order_ptr, order_dev = _order(dispatch_order, B, dev)
    rc = lib().pa_decode_gqa(_ptr(out), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables), _ptr(context_lens),
                             B, int(block_tables.shape[1]), num_pages, int(page_size), float(scale), odt,
                             _ptr(workspace), ws_bytes, _ptr(device_flags), order_ptr, order_dev, _stream(stream))
    _check(rc, "pa_decode_gqa")
    return out


def append_decode_gqa(out: torch.Tensor, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                      k_pool: torch.Tensor, v_pool: torch.Tensor, block_tables: torch.Tensor,
                      context_lens: torch.Tensor, rope_cos_sin: torch.Tensor, scale: float = 0.125,
                      workspace: Optional[torch.Tensor] = None, device_flags: Optional[torch.Tensor] = None,
                      page_size: int = 16, dispatch_order=None, stream=None) -> torch.Tensor:
    """pa_append_decode_gqa: append (RoPE K, V at pos = L-1), rotate q in place, then decode into ``out``."""
    num_pages = _pool_checks(k_pool, v_pool)
    dev = k_pool.device
    _expect(context_lens, "context_lens", torch.int32, device=dev)
    B = int(context_lens.shape[0])
    _expect(block_tables, "block_tables", torch.int32, device=dev)
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [num_seqs][max_blocks]")
    _expect(q, "q", torch.bfloat16, (B, 32, 64), dev)
    _expect(k_new, "k_new", torch.bfloat16, (B, 8, 64), dev)
    _expect(v_new, "v_new", torch.bfloat16, (B, 8, 64), dev)
    _expect(rope_cos_sin, "rope_cos_sin", torch.float64, device=dev)
    if out.dtype == torch.bfloat16:
        odt = PA_OUT_BF16
    elif out.dtype == torch.float32:
        odt = PA_OUT_FP32
    else:
        raise TypeError("out must be bfloat16 or float32")
    _expect(out, "out", out.dtype, (B, 32, 64), dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if device_flags is not None:
        _expect(device_flags, "device_flags", torch.int32, (1,), dev)
    order_keep, order_ptr, order_dev = _order(dispatch_order, B, dev)
    rc = lib().pa_append_decode_gqa(_ptr(out), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_pool), _ptr(v_pool),
                                    _ptr(block_tables), _ptr(context_lens), _ptr(rope_cos_sin), B,
                                    int(block_tables.shape[1]), num_pages, int(page_size), int(rope_cos_sin.shape[0]),
                                    float(scale), odt, _ptr(workspace), ws_bytes, _ptr(device_flags), order_ptr,
                                    order_dev, _stream(stream))
    _check(rc, "pa_append_decode_gqa")
    return out


NOALLOC_SCRATCH_BYTES = 8 << 20  # PA_NOALLOC_SCRATCH_BYTES


def append_decode_gqa_noalloc(out: torch.Tensor, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                              k_pool: torch.Tensor, v_pool: torch.Tensor, block_tables: torch.Tensor,
                              context_lens: torch.Tensor, rope_cos_sin: torch.Tensor, scale: float = 0.125,
                              device_flags: Optional[torch.Tensor] = None, page_size: int = 16,
                              dispatch_order=None, stream=None) -> torch.Tensor:
    """pa_append_decode_gqa_noalloc: pa_append_decode_gqa with the library's own per-GPU scratch
    in place of a workspace (nothing is allocated; calls on one GPU must not overlap)."""
    num_pages = _pool_checks(k_pool, v_pool)
    dev = k_pool.device
    _expect(context_lens, "context_lens", torch.int32, device=dev)
    B = int(context_lens.shape[0])
    _expect(block_tables, "block_tables", torch.int32, device=dev)
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [num_seqs][max_blocks]")
    _expect(q, "q", torch.bfloat16, (B, 32, 64), dev)
    _expect(k_new, "k_new", torch.bfloat16, (B, 8, 64), dev)
    _expect(v_new, "v_new", torch.bfloat16, (B, 8, 64), dev)
    _expect(rope_cos_sin, "rope_cos_sin", torch.float64, device=dev)
    odt = _out_dtype(out)
    _expect(out, "out", out.dtype, (B, 32, 64), dev)
    if device_flags is not None:
        _expect(device_flags, "device_flags", torch.int32, (1,), dev)
    order_keep, order_ptr, order_dev = _order(dispatch_order, B, dev)
    rc = lib().pa_append_decode_gqa_noalloc(_ptr(out), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_pool),
                                            _ptr(v_pool), _ptr(block_tables), _ptr(context_lens),
                                            _ptr(rope_cos_sin), B, int(block_tables.shape[1]), num_pages,
                                            int(page_size), int(rope_cos_sin.shape[0]), float(scale), odt,
                                            _ptr(device_flags), order_ptr, order_dev, _stream(stream))
    _check(rc, "pa_append_decode_gqa_noalloc")
    return out


def prefill_chunk(out: torch.Tensor, q: torch.Tensor, k_chunk: torch.Tensor, v_chunk: torch.Tensor,
                  k_pool: torch.Tensor, v_pool: torch.Tensor, block_tables: torch.Tensor, prefix_lens: torch.Tensor,
                  rope_cos_sin: torch.Tensor, scale: float = 0.125, device_flags: Optional[torch.Tensor] = None,
                  page_size: int = 16, stream=None) -> torch.Tensor:
    """pa_prefill_chunk: append the chunk (q rotated in place), then causal paged attention into ``out``."""
    num_pages = _pool_checks(k_pool, v_pool)
    dev = k_pool.device
    _expect(prefix_lens, "prefix_lens", torch.int32, device=dev)
    B = int(prefix_lens.shape[0])
    if q.dim() != 4:
        raise ValueError("q must be [num_seqs][chunk_len][32][64]")
    C = int(q.shape[1])
    _expect(q, "q", torch.bfloat16, (B, C, 32, 64), dev)
    _expect(k_chunk, "k_chunk", torch.bfloat16, (B, C, 8, 64), dev)
    _expect(v_chunk, "v_chunk", torch.bfloat16, (B, C, 8, 64), dev)
    _expect(block_tables, "block_tables", torch.int32, device=dev)
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [num_seqs][max_blocks]")
    _expect(rope_cos_sin, "rope_cos_sin", torch.float64, device=dev)
    if out.dtype == torch.bfloat16:
        odt = PA_OUT_BF16
    elif out.dtype == torch.float32:
        odt = PA_OUT_FP32
    else:
        raise TypeError("out must be bfloat16 or float32")
    _expect(out, "out", out.dtype, (B, C, 32, 64), dev)
    if device_flags is not None:
        _expect(device_flags, "device_flags", torch.int32, (1,), dev)
    rc = lib().pa_prefill_chunk(_ptr(out), _ptr(q), _ptr(k_chunk), _ptr(v_chunk), _ptr(k_pool), _ptr(v_pool),
                                _ptr(block_tables), _ptr(prefix_lens), _ptr(rope_cos_sin), B, C,
                                int(block_tables.shape[1]), num_pages, int(page_size), int(rope_cos_sin.shape[0]),
                                float(scale), odt, _ptr(device_flags), _stream(stream))
    _check(rc, "pa_prefill_chunk")
    return out


# ------------------------------------------------------------ INT8 pages --

def i8_pool(num_pages: int, device="cuda") -> torch.Tensor:
    """An (uninitialised) INT8 pool: uint8 [num_pages][8][2176] (pa_i8_pool_bytes bytes)."""
    n = int(lib().pa_i8_pool_bytes(int(num_pages)))
    if n == 0:
        raise ValueError("num_pages must be positive")
    return torch.empty((int(num_pages), _w.NUM_KV_HEADS, PA_I8_TILE_BYTES), dtype=torch.uint8, device=device)


def _i8_pool_checks(pool):
    _expect(pool, "kv_pool_i8", torch.uint8)
    if pool.dim() != 3 or tuple(pool.shape[1:]) != (_w.NUM_KV_HEADS, PA_I8_TILE_BYTES):
        raise ValueError(f"INT8 pool must be [num_pages][8][2176] uint8, got {tuple(pool.shape)}")
    return int(pool.shape[0])


def prefill_chunk_i8(out: torch.Tensor, q: torch.Tensor, k_chunk: torch.Tensor, v_chunk: torch.Tensor,
                     kv_pool_i8: torch.Tensor, block_tables: torch.Tensor, prefix_lens: torch.Tensor,
                     rope_cos_sin: torch.Tensor, scale: float = 0.125, device_flags: Optional[torch.Tensor] = None,
                     page_size: int = 16, stream=None) -> torch.Tensor:
    """pa_prefill_chunk_i8: quantise the chunk into the INT8 pool (q rotated in place), then causal
    attention over the INT8 pages into ``out``."""
    num_pages = _i8_pool_checks(kv_pool_i8)
    dev = kv_pool_i8.device
    _expect(prefix_lens, "prefix_lens", torch.int32, device=dev)
    B = int(prefix_lens.shape[0])
    if q.dim() != 4:
        raise ValueError("q must be [num_seqs][chunk_len][32][64]")
    C = int(q.shape[1])
    _expect(q, "q", torch.bfloat16, (B, C, 32, 64), dev)
    _expect(k_chunk, "k_chunk", torch.bfloat16, (B, C, 8, 64), dev)
    _expect(v_chunk, "v_chunk", torch.bfloat16, (B, C, 8, 64), dev)
    _expect(block_tables, "block_tables", torch.int32, device=dev)
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [num_seqs][max_blocks]")
    _expect(rope_cos_sin, "rope_cos_sin", torch.float64, device=dev)
    odt = _out_dtype(out)
    _expect(out, "out", out.dtype, (B, C, 32, 64), dev)
    if device_flags is not None:
        _expect(device_flags, "device_flags", torch.int32, (1,), dev)
    rc = lib().pa_prefill_chunk_i8(_ptr(out), _ptr(q), _ptr(k_chunk), _ptr(v_chunk), _ptr(kv_pool_i8),
                                   _ptr(block_tables), _ptr(prefix_lens), _ptr(rope_cos_sin), B, C,
                                   int(block_tables.shape[1]), num_pages, int(page_size), int(rope_cos_sin.shape[0]),
                                   float(scale), odt, _ptr(device_flags), _stream(stream))
    _check(rc, "pa_prefill_chunk_i8")
    return out


def _tables(block_tables, context_lens, dev):
    _expect(context_lens, "context_lens", torch.int32, device=dev)
    B = int(context_lens.shape[0])
    _expect(block_tables, "block_tables", torch.int32, device=dev)
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [num_seqs][max_blocks]")
    return B


def _out_dtype(out):
    if out.dtype == torch.bfloat16:
        return PA_OUT_BF16
    if out.dtype == torch.float32:
        return PA_OUT_FP32
    raise TypeError("out must be bfloat16 or float32")


def quantize_pages_i8(kv_pool_i8: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                      page_ids: Optional[torch.Tensor] = None, device_flags: Optional[torch.Tensor] = None,
                      stream=None) -> None:
    """pa_quantize_pages_i8: quantise the listed bf16 pages (all when page_ids is None) into the INT8 pool."""
    num_pages = _i8_pool_checks(kv_pool_i8)
    if _pool_checks(k_pool, v_pool) != num_pages:
        raise ValueError("bf16 pools and the INT8 pool must have the same number of pages")
    dev = kv_pool_i8.device
    if page_ids is not None:
        _expect(page_ids, "page_ids", torch.int32, device=dev)
        count = int(page_ids.numel())
    else:
        count = num_pages
    if device_flags is not None:
        _expect(device_flags, "device_flags", torch.int32, (1,), dev)
    _check(lib().pa_quantize_pages_i8(_ptr(kv_pool_i8), _ptr(k_pool), _ptr(v_pool), _ptr(page_ids), count, num_pages,
                                      _ptr(device_flags), _stream(stream)), "pa_quantize_pages_i8")


def append_kv_rope_i8(q: Optional[torch.Tensor], k_new: torch.Tensor, v_new: torch.Tensor, kv_pool_i8: torch.Tensor,
                      block_tables: torch.Tensor, context_lens: torch.Tensor, rope_cos_sin: torch.Tensor,
                      device_flags: Optional[torch.Tensor] = None, page_size: int = 16, stream=None) -> None:
    """pa_append_kv_rope_i8: quantise RoPE(k_new) and v_new into slot pos = L-1; rotate q in place (if given)."""
    num_pages = _i8_pool_checks(kv_pool_i8)
    dev = kv_pool_i8.device
    B = _tables(block_tables, context_lens, dev)
    _expect(k_new, "k_new", torch.bfloat16, (B, 8, 64), dev)
    _expect(v_new, "v_new", torch.bfloat16, (B, 8, 64), dev)
    if q is not None:
        _expect(q, "q", torch.bfloat16, (B, 32, 64), dev)
    _expect(rope_cos_sin, "rope_cos_sin", torch.float64, device=dev)
    if device_flags is not None:
        _expect(device_flags, "device_flags", torch.int32, (1,), dev)
    rc = lib().pa_append_kv_rope_i8(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(kv_pool_i8), _ptr(block_tables),
                                    _ptr(context_lens), _ptr(rope_cos_sin), B, int(block_tables.shape[1]), num_pages,
                                    int(page_size), int(rope_cos_sin.shape[0]), _ptr(device_flags), _stream(stream))
    _check(rc, "pa_append_kv_rope_i8")


def decode_gqa_i8(out: torch.Tensor, q: torch.Tensor, kv_pool_i8: torch.Tensor, block_tables: torch.Tensor,
                  context_lens: torch.Tensor, scale: float = 0.125, workspace: Optional[torch.Tensor] = None,
                  device_flags: Optional[torch.Tensor] = None, page_size: int = 16, dispatch_order=None,
                  stream=None) -> torch.Tensor:
    """pa_decode_gqa_i8 into ``out`` ([B][32][64] bf16 or fp32; may be ``q`` itself)."""
    num_pages = _i8_pool_checks(kv_pool_i8)
    dev = kv_pool_i8.device
    B = _tables(block_tables, context_lens, dev)
    _expect(q, "q", torch.bfloat16, (B, 32, 64), dev)
    odt = _out_dtype(out)
    _expect(out, "out", out.dtype, (B, 32, 64), dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if device_flags is not None:
        _expect(device_flags, "device_flags", torch.int32, (1,), dev)
    order_keep, order_ptr, order_dev = _order(dispatch_order, B, dev)
    rc = lib().pa_decode_gqa_i8(_ptr(out), _ptr(q), _ptr(kv_pool_i8), _ptr(block_tables), _ptr(context_lens), B,
                                int(block_tables.shape[1]), num_pages, int(page_size), float(scale), odt,
                                _ptr(workspace), ws_bytes, _ptr(device_flags), order_ptr, order_dev, _stream(stream))
    _check(rc, "pa_decode_gqa_i8")
    return out


def append_decode_gqa_i8(out: torch.Tensor, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                         kv_pool_i8: torch.Tensor, block_tables: torch.Tensor, context_lens: torch.Tensor,
                         rope_cos_sin: torch.Tensor, scale: float = 0.125, workspace: Optional[torch.Tensor] = None,
                         device_flags: Optional[torch.Tensor] = None, page_size: int = 16,
                         dispatch_order=None, stream=None) -> torch.Tensor:
    """pa_append_decode_gqa_i8: quantised append at pos = L-1, q rotated in place, then decode into ``out``."""
    num_pages = _i8_pool_checks(kv_pool_i8)
    dev = kv_pool_i8.device
    B = _tables(block_tables, context_lens, dev)
    _expect(q, "q", torch.bfloat16, (B, 32, 64), dev)
    _expect(k_new, "k_new", torch.bfloat16, (B, 8, 64), dev)
    _expect(v_new, "v_new", torch.bfloat16, (B, 8, 64), dev)
    _expect(rope_cos_sin, "rope_cos_sin", torch.float64, device=dev)
    odt = _out_dtype(out)
    _expect(out, "out", out.dtype, (B, 32, 64), dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if device_flags is not None:
        _expect(device_flags, "device_flags", torch.int32, (1,), dev)
    order_keep, order_ptr, order_dev = _order(dispatch_order, B, dev)
    rc = lib().pa_append_decode_gqa_i8(_ptr(out), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(kv_pool_i8),
                                       _ptr(block_tables), _ptr(context_lens), _ptr(rope_cos_sin), B,
                                       int(block_tables.shape[1]), num_pages, int(page_size),
                                       int(rope_cos_sin.shape[0]), float(scale), odt, _ptr(workspace), ws_bytes,
                                       _ptr(device_flags), order_ptr, order_dev, _stream(stream))
    _check(rc, "pa_append_decode_gqa_i8")
    return out


# ----------------------------------------------------------------- argmax --

def argmax_workspace(num_rows: int, vocab: int, dtype: torch.dtype, device="cuda") -> Optional[torch.Tensor]:
    code = PA_LOGITS_BF16 if dtype == torch.bfloat16 else PA_LOGITS_FP32
    n = int(lib().pa_argmax_workspace_bytes(int(num_rows), int(vocab), code))
    # zeroed once here; every pa_argmax call leaves it zeroed again
    return None if n == 0 else torch.zeros(n // 8, dtype=torch.int64, device=device)


def argmax(out_index: torch.Tensor, logits: torch.Tensor, workspace: Optional[torch.Tensor] = None,
           stream=None) -> torch.Tensor:
    """pa_argmax: out_index[r] = lowest index of the row's non-NaN maximum (0 for an all-NaN row)."""
    if logits.dim() != 2:
        raise ValueError("logits must be [num_rows][vocab]")
    if logits.dtype == torch.bfloat16:
        code = PA_LOGITS_BF16
    elif logits.dtype == torch.float32:
        code = PA_LOGITS_FP32
    else:
        raise TypeError("logits must be bfloat16 or float32")
    _expect(logits, "logits", logits.dtype)
    rows, vocab = int(logits.shape[0]), int(logits.shape[1])
    _expect(out_index, "out_index", torch.int32, (rows,), logits.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().pa_argmax(_ptr(out_index), _ptr(logits), rows, vocab, code, _ptr(workspace), ws_bytes,
                           _stream(stream)), "pa_argmax")
    return out_index


def dispatch_order_longest_first(lengths) -> np.ndarray:
    """pa_dispatch_order_longest_first: batch indices by length, longest first (stable), as the
    int32 array the decode calls take as dispatch_order."""
    lens = np.ascontiguousarray(np.asarray(lengths, dtype=np.int32))
    order = np.empty(lens.shape[0], dtype=np.int32)
    _check(lib().pa_dispatch_order_longest_first(ctypes.c_void_p(lens.ctypes.data), int(lens.shape[0]),
                                                 ctypes.c_void_p(order.ctypes.data)),
           "pa_dispatch_order_longest_first")
    return order


def order_by_length(context_lens: torch.Tensor, max_blocks: int, order: Optional[torch.Tensor] = None,
                    long_run: int = 1, short_run: int = 0, stream=None) -> torch.Tensor:
    """pa_order_by_length: the sequences ranked longest first (64 length classes across
    max_blocks pages, index order within a class) and dealt in runs of ``long_run`` from the
    long end and ``short_run`` from the short end, computed on the device into ``order``
    (int32[num_seqs], a new tensor when None).  Pass it as ``dispatch_order`` to the decode calls
    of the step."""
    _expect(context_lens, "context_lens", torch.int32)
    if context_lens.dim() != 1:
        raise ValueError("context_lens must be [num_seqs]")
    n = int(context_lens.shape[0])
    if order is None:
        order = torch.empty(n, dtype=torch.int32, device=context_lens.device)
    _expect(order, "order", torch.int32, (n,), context_lens.device)
    _check(lib().pa_order_by_length(_ptr(context_lens), n, int(max_blocks), int(long_run), int(short_run),
                                    _ptr(order), _stream(stream)), "pa_order_by_length")
    return order


def probe_stream_read(buf: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """pa_probe_stream_read: read all of buf's bytes once (a contiguous-read bandwidth probe)."""
    if not isinstance(buf, torch.Tensor) or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous tensor")
    _expect(sink, "sink", torch.int32, (1,), buf.device)
    nbytes = buf.numel() * buf.element_size()
    _check(lib().pa_probe_stream_read(_ptr(buf), nbytes, _ptr(sink), _stream(stream)), "pa_probe_stream_read")


def admission_credit_pages(prompt_tokens: int, max_new_tokens: int, num_layers: int) -> int:
    return int(lib().pa_admission_credit_pages(int(prompt_tokens), int(max_new_tokens), int(num_layers)))


class KVManager:
    """Host page manager of libpa (pa_kvm_*): free list, per-(slot, layer) block
    tables, admission credit and batching policy.  Thin wrapper: every decision
    is made by the library; this class only copies its tables into numpy."""

    def __init__(self, num_pages: int, num_layers: int, max_slots: int, max_blocks: int,
                 batching: int = PA_BATCH_CONTINUOUS):
        self.num_pages, self.num_layers = int(num_pages), int(num_layers)
        self.max_slots, self.max_blocks = int(max_slots), int(max_blocks)
        h = ctypes.c_void_p()
        _check(lib().pa_kvm_create(self.num_pages, self.num_layers, self.max_slots, self.max_blocks, int(batching),
                                   ctypes.byref(h)), "pa_kvm_create")
        self._h = h

    def close(self) -> None:
        if getattr(self, "_h", None):
            lib().pa_kvm_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def submit(self, prompt_tokens: int, max_new_tokens: int) -> int:
        rid = ctypes.c_int32(-1)
        _check(lib().pa_kvm_submit(self._h, int(prompt_tokens), int(max_new_tokens), ctypes.byref(rid)),
               "pa_kvm_submit")
        return int(rid.value)

    def schedule(self, max_out: Optional[int] = None) -> list:
        n_max = self.max_slots if max_out is None else int(max_out)
        buf = (ctypes.c_int32 * max(n_max, 1))()
        n = int(lib().pa_kvm_schedule(self._h, buf, n_max))
        if n < 0:
            raise PaError(PA_ERR_INVALID_ARG, "pa_kvm_schedule")
        return [int(buf[i]) for i in range(n)]

    def set_length(self, slot: int, length: int) -> None:
        _check(lib().pa_kvm_set_length(self._h, int(slot), int(length)), "pa_kvm_set_length")

    def release(self, slot: int) -> None:
        _check(lib().pa_kvm_release(self._h, int(slot)), "pa_kvm_release")

    def block_tables(self) -> np.ndarray:
        """Copy of the tables, [num_layers][max_slots][max_blocks] int32."""
        n = self.num_layers * self.max_slots * self.max_blocks
        p = lib().pa_kvm_block_tables(self._h)
        return np.ctypeslib.as_array(p, shape=(n,)).reshape(self.num_layers, self.max_slots,
                                                             self.max_blocks).copy()

    def lengths(self) -> np.ndarray:
        p = lib().pa_kvm_lengths(self._h)
        return np.ctypeslib.as_array(p, shape=(self.max_slots,)).copy()

    def slot_request(self, slot: int) -> int:
        return int(lib().pa_kvm_slot_request(self._h, int(slot)))

    def slot_budget(self, slot: int) -> int:
        return int(lib().pa_kvm_slot_budget(self._h, int(slot)))

    @property
    def free_pages(self) -> int:
        return int(lib().pa_kvm_free_pages(self._h))

    @property
    def reserved_pages(self) -> int:
        return int(lib().pa_kvm_reserved_pages(self._h))

    @property
    def queued(self) -> int:
        return int(lib().pa_kvm_queued(self._h))
