"""fp64 CPU oracle for paged GQA decode, KV append + RoPE and chunked prefill.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The library under
``paged_kv_gqa_append_amd`` never imports, links or calls it, and it shares no
code with the HIP path: the arithmetic lives in ``oracle.c`` (plain loops,
double precision), this file only marshals numpy arrays through ctypes.

Inputs are numpy arrays: bf16 tensors as ``uint16`` bit patterns, page tables
and lengths as ``int32``.  Layouts: see ``oracle.c``.

Pins (tests/test_oracle_*.py): bf16 rounding against torch's float32 -> bf16
and hand-built halfway cases; RoPE against complex multiplication and the
Hugging Face Llama rotate-half routine; decode against torch's fp64
``scaled_dot_product_attention`` on gathered contiguous K/V plus closed forms
(single token, identical rows, q = 0, two-token logistic, ones column) and
page-placement invariance; prefill against causal SDPA and decode; the INT8
prefill (a composition of the INT8 append and decode) against causal SDPA on
the dequantised pool and against the bf16 prefill's rows quantised.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
# A test may point the wrapper at another build of an oracle.c copy (the mutation sweep
# in tests/test_oracle_mutation.py); that library is loaded as it is, never rebuilt.
_OVERRIDE = os.environ.get("PA_ORACLE_LIB")
_lib = None

CFLAGS = ["-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra", "-fno-fast-math",
          "-ffp-contract=off"]


def compile_c(src: str, out: str) -> str:
    """gcc src (an oracle.c) into the shared library out, with the oracle's flags."""
    tmp = out + ".tmp"
    subprocess.run(["gcc", *CFLAGS, src, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, out)
    return out

OK, BAD_ARG, BAD_LEN, BAD_PAGE = 0, 1, 2, 3


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (-O2, OpenMP) into oracle/liboracle.so."""
    if force or not os.path.exists(_LIB_PATH):
        compile_c(_SRC, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if _OVERRIDE:
        lib = ctypes.CDLL(_OVERRIDE)
    else:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i32 = ctypes.c_int32
    dbl = ctypes.c_double
    lib.oracle_bf16_to_f64.restype = dbl
    lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_f64_to_bf16.restype = ctypes.c_uint16
    lib.oracle_f64_to_bf16.argtypes = [dbl]
    lib.oracle_rope_head.restype = None
    lib.oracle_rope_head.argtypes = [P, ctypes.c_int64, dbl, P]
    lib.oracle_append_kv_rope.restype = ctypes.c_int
    lib.oracle_append_kv_rope.argtypes = [P, P, P, P, P, P, P, i32, i32, i32, dbl]
    lib.oracle_decode_gqa.restype = ctypes.c_int
    lib.oracle_decode_gqa.argtypes = [P, P, P, P, P, P, i32, i32, i32, dbl]
    lib.oracle_prefill_chunk.restype = ctypes.c_int
    lib.oracle_prefill_chunk.argtypes = [P, P, P, P, P, P, P, P, i32, i32, i32, i32, dbl, dbl]
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    _lib = lib
    return lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError(f"bf16 tensors are passed as uint16 bit patterns, got {a.dtype}")
    return a


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.int32)


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def bf16_to_f64(b: int) -> float:
    return float(_load().oracle_bf16_to_f64(int(b)))


def f64_to_bf16(x: float) -> int:
    """One-step round-to-nearest-even of a double to bf16 (bit pattern)."""
    return int(_load().oracle_f64_to_bf16(float(x)))


def rope_head(x_bits: np.ndarray, pos: int, theta: float) -> np.ndarray:
    """Rotate one 64-wide bf16 head to fp64 at absolute position ``pos``."""
    x = _u16(x_bits)
    assert x.shape == (64,)
    y = np.zeros(64, dtype=np.float64)
    _load().oracle_rope_head(_ptr(x), int(pos), float(theta), _ptr(y))
    return y


def append_kv_rope(q, k_new, v_new, k_pool, v_pool, block_tables, context_lens, num_pages: int,
                   theta: float) -> int:
    """In place on ``q`` (may be None), ``k_pool`` and ``v_pool``; returns a status code."""
    lib = _load()
    qq = None if q is None else _u16(q)
    for a in (k_pool, v_pool) + (() if q is None else (q,)):
        if not (a.flags.c_contiguous and a.dtype == np.uint16):
            raise TypeError("in-place arrays must be C-contiguous uint16")
    kn, vn = _u16(k_new), _u16(v_new)
    bt, cl = _i32(block_tables), _i32(context_lens)
    B = int(cl.shape[0])
    return int(lib.oracle_append_kv_rope(_ptr(qq), _ptr(kn), _ptr(vn), _ptr(k_pool), _ptr(v_pool), _ptr(bt),
                                         _ptr(cl), B, int(bt.shape[-1]), int(num_pages), float(theta)))


def decode_gqa(q, k_pool, v_pool, block_tables, context_lens, num_pages: int, scale: float):
    """Returns (out fp64 [B][32][64], status)."""
    lib = _load()
    qq, kp, vp = _u16(q), _u16(k_pool), _u16(v_pool)
    bt, cl = _i32(block_tables), _i32(context_lens)
    B = int(cl.shape[0])
    out = np.zeros((B, 32, 64), dtype=np.float64)
    rc = lib.oracle_decode_gqa(_ptr(out), _ptr(qq), _ptr(kp), _ptr(vp), _ptr(bt), _ptr(cl), B,
                               int(bt.shape[-1]), int(num_pages), float(scale))
    return out, int(rc)


def prefill_chunk(q, k_chunk, v_chunk, k_pool, v_pool, block_tables, prefix_lens, num_pages: int,
                  theta: float, scale: float):
    """In place on ``q``, ``k_pool``, ``v_pool``; returns (out fp64 [B][C][32][64], status)."""
    lib = _load()
    for a in (q, k_pool, v_pool):
        if not (a.flags.c_contiguous and a.dtype == np.uint16):
            raise TypeError("in-place arrays must be C-contiguous uint16")
    kc, vc = _u16(k_chunk), _u16(v_chunk)
    bt, pl = _i32(block_tables), _i32(prefix_lens)
    B, C = int(q.shape[0]), int(q.shape[1])
    out = np.zeros((B, C, 32, 64), dtype=np.float64)
    rc = lib.oracle_prefill_chunk(_ptr(out), _ptr(q), _ptr(kc), _ptr(vc), _ptr(k_pool), _ptr(v_pool), _ptr(bt),
                                  _ptr(pl), B, C, int(bt.shape[-1]), int(num_pages), float(theta), float(scale))
    return out, int(rc)


# ------------------------------------------------------------------ INT8 pages --
I8_TILE_BYTES = 2176


def _i8_setup(lib):
    P, i32, dbl = ctypes.c_void_p, ctypes.c_int32, ctypes.c_double
    lib.oracle_quantize_row_i8.restype = None
    lib.oracle_quantize_row_i8.argtypes = [P, P, P]
    lib.oracle_append_kv_rope_i8.restype = ctypes.c_int
    lib.oracle_append_kv_rope_i8.argtypes = [P, P, P, P, P, P, i32, i32, i32, dbl]
    lib.oracle_decode_gqa_i8.restype = ctypes.c_int
    lib.oracle_decode_gqa_i8.argtypes = [P, P, P, P, P, i32, i32, i32, dbl]
    lib.oracle_quantize_pages_i8.restype = None
    lib.oracle_quantize_pages_i8.argtypes = [P, P, P, i32]


def quantize_row_i8(x_bits):
    """One 64-value row (bf16 patterns) -> (int8 codes [64], fp32 scale)."""
    lib = _load()
    _i8_setup(lib)
    x = _u16(x_bits)
    assert x.shape == (64,)
    codes = np.zeros(64, dtype=np.int8)
    sc = np.zeros(1, dtype=np.float32)
    lib.oracle_quantize_row_i8(_ptr(x), _ptr(codes), _ptr(sc))
    return codes, np.float32(sc[0])


def quantize_pages_i8(k_pool, v_pool, pool=None):
    """bf16 pools [P][8][16][64] -> INT8 pool uint8 [P][8][2176] (rows with a
    non-finite value keep the bytes ``pool`` had; a fresh pool starts zeroed)."""
    lib = _load()
    _i8_setup(lib)
    kp, vp = _u16(k_pool), _u16(v_pool)
    assert kp.shape == vp.shape and kp.shape[1:] == (8, 16, 64)
    P = int(kp.shape[0])
    if pool is None:
        pool = np.zeros((P, 8, 2176), dtype=np.uint8)
    if not (pool.flags.c_contiguous and pool.dtype == np.uint8 and pool.shape == (P, 8, 2176)):
        raise TypeError("pool must be C-contiguous uint8 [P][8][2176]")
    lib.oracle_quantize_pages_i8(_ptr(pool), _ptr(kp), _ptr(vp), P)
    return pool


def append_kv_rope_i8(q, k_new, v_new, pool, block_tables, context_lens, num_pages: int, theta: float) -> int:
    """In place on ``q`` (may be None) and ``pool`` (uint8 [P][8][2176]); returns a status code."""
    lib = _load()
    _i8_setup(lib)
    if not (pool.flags.c_contiguous and pool.dtype == np.uint8):
        raise TypeError("pool must be C-contiguous uint8")
    if q is not None and not (q.flags.c_contiguous and q.dtype == np.uint16):
        raise TypeError("q must be C-contiguous uint16")
    kn, vn = _u16(k_new), _u16(v_new)
    bt, cl = _i32(block_tables), _i32(context_lens)
    return int(lib.oracle_append_kv_rope_i8(_ptr(q), _ptr(kn), _ptr(vn), _ptr(pool), _ptr(bt), _ptr(cl),
                                            int(cl.shape[0]), int(bt.shape[-1]), int(num_pages), float(theta)))


def decode_gqa_i8(q, pool, block_tables, context_lens, num_pages: int, scale: float):
    """Returns (out fp64 [B][32][64], status)."""
    lib = _load()
    _i8_setup(lib)
    qq = _u16(q)
    pl = np.ascontiguousarray(pool, dtype=np.uint8)
    bt, cl = _i32(block_tables), _i32(context_lens)
    B = int(cl.shape[0])
    out = np.zeros((B, 32, 64), dtype=np.float64)
    rc = lib.oracle_decode_gqa_i8(_ptr(out), _ptr(qq), _ptr(pl), _ptr(bt), _ptr(cl), B, int(bt.shape[-1]),
                                  int(num_pages), float(scale))
    return out, int(rc)


def prefill_chunk_i8(q, k_chunk, v_chunk, pool, block_tables, prefix_lens, num_pages: int, theta: float,
                     scale: float):
    """Chunked prefill into INT8 pages (TinyLoop, "prefill_chunk and scratch residency": the prompt in
    row chunks; "Per-request / handle-owned memory": the INT8 K/V mode), written as what it is made of:
    chunk token i of every sequence is appended at position prefix + i exactly as ``append_kv_rope_i8``
    appends one token (its decode length prefix + i + 1), q row i rotated with it; then chunk row i
    attends causally, keys 0 .. prefix + i, exactly as ``decode_gqa_i8`` at that length.  In place on
    ``q`` (uint16 [B][C][32][64]) and ``pool``; returns (out fp64 [B][C][32][64], status)."""
    if not (q.flags.c_contiguous and q.dtype == np.uint16):
        raise TypeError("q must be C-contiguous uint16")
    kc, vc = _u16(k_chunk), _u16(v_chunk)
    pl = _i32(prefix_lens).astype(np.int64)
    B, C = int(q.shape[0]), int(q.shape[1])
    rc = OK
    for i in range(C):
        qi = np.ascontiguousarray(q[:, i])
        r = append_kv_rope_i8(qi, kc[:, i], vc[:, i], pool, block_tables, (pl + i + 1).astype(np.int32), num_pages,
                              theta)
        q[:, i] = qi
        rc = rc if rc != OK else r
    out = np.zeros((B, C, 32, 64), dtype=np.float64)
    for i in range(C):
        o, r = decode_gqa_i8(q[:, i], pool, block_tables, (pl + i + 1).astype(np.int32), num_pages, scale)
        out[:, i] = o
        rc = rc if rc != OK else r
    return out, rc


def argmax(logits) -> np.ndarray:
    """Lowest index of the row maximum over non-NaN entries (0 for an all-NaN
    row).  ``logits``: [rows][vocab] as uint16 bf16 patterns or float32."""
    lib = _load()
    lib.oracle_argmax.restype = ctypes.c_int
    lib.oracle_argmax.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int]
    x = np.ascontiguousarray(logits)
    if x.ndim != 2 or x.dtype not in (np.uint16, np.float32):
        raise TypeError("logits must be 2-D uint16 (bf16 patterns) or float32")
    out = np.zeros(x.shape[0], dtype=np.int32)
    rc = lib.oracle_argmax(_ptr(out), _ptr(x), int(x.shape[0]), int(x.shape[1]), int(x.dtype == np.uint16))
    if rc != OK:
        raise ValueError(f"oracle_argmax: status {rc}")
    return out
