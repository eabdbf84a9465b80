"""Host-side checks of libpa.so that need no GPU.

* every function include/pa.h declares is exported;
* host validation returns its status before any launch (so these calls are
  safe without a device: each one is invalid in some host-visible way);
* workspace sizing and the fp64 -> fp32 RoPE table builder.
"""
import ctypes
import math
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pa.h")


@pytest.fixture(scope="module")
def pa():
    from paged_kv_gqa_append_amd import binding, build

    if not build.is_current():
        build.build()
    binding.lib()
    return binding


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(pa):
    names = declared_functions()
    assert set(names) >= {"pa_append_kv_rope", "pa_decode_gqa", "pa_prefill_chunk"}
    lib = pa.lib()
    for n in names:
        assert hasattr(lib, n), f"libpa.so does not export {n}"
    assert set(pa.EXPORTS) == set(names)


def test_status_strings(pa):
    assert pa.status_string(0) == "PA_OK"
    assert pa.status_string(3) == "PA_ERR_WORKSPACE"
    assert pa.status_string(99) == "PA_ERR_UNKNOWN"
    assert pa.lib().pa_abi_version() == pa.ABI_VERSION == 14


FAKE = 0x7F0000000000  # never dereferenced: every call below fails validation first


def decode_call(lib, out=FAKE, q=FAKE, kp=FAKE, vp=FAKE, bt=FAKE, cl=FAKE, B=4, mb=8, P=64, ps=16, scale=0.125,
                odt=0, ws=None, wsb=0, order=None, dorder=None):
    v = ctypes.c_void_p
    op = None if order is None else np.ascontiguousarray(order, dtype=np.int32).ctypes.data_as(v)
    return lib.pa_decode_gqa(v(out), v(q), v(kp), v(vp), v(bt), v(cl), B, mb, P, ps, scale, odt, v(ws) if ws else None,
                             wsb, None, op, v(dorder) if dorder else None, None)


def test_decode_validation(pa):
    lib = pa.lib()
    assert decode_call(lib, ps=32) == pa.PA_ERR_UNSUPPORTED
    assert decode_call(lib, odt=7) == pa.PA_ERR_UNSUPPORTED
    assert decode_call(lib, B=-1) == pa.PA_ERR_INVALID_ARG
    assert decode_call(lib, mb=0) == pa.PA_ERR_INVALID_ARG
    assert decode_call(lib, P=0) == pa.PA_ERR_INVALID_ARG
    assert decode_call(lib, scale=float("nan")) == pa.PA_ERR_INVALID_ARG
    assert decode_call(lib, q=0) == pa.PA_ERR_INVALID_ARG
    assert decode_call(lib, out=FAKE + 8) == pa.PA_ERR_INVALID_ARG
    assert decode_call(lib, kp=FAKE + 2) == pa.PA_ERR_INVALID_ARG
    # an empty batch is a no-op, whatever the pointers
    assert decode_call(lib, B=0, q=0, out=0) == pa.PA_OK
    # long tables need a workspace
    mb = 128
    need = lib.pa_decode_workspace_bytes(4, mb)
    if need:
        assert decode_call(lib, mb=mb) == pa.PA_ERR_WORKSPACE
        assert decode_call(lib, mb=mb, ws=FAKE, wsb=need - 4) == pa.PA_ERR_WORKSPACE
        assert decode_call(lib, mb=mb, ws=FAKE + 4, wsb=need) == pa.PA_ERR_WORKSPACE


def test_dispatch_order_validation(pa):
    """A dispatch order must be a permutation of the batch and fit the launch
    arguments (sequences x partitions <= PA_MAX_DISPATCH_ORDER, at most 64
    partitions); otherwise the call is refused before anything is launched."""
    lib = pa.lib()
    for bad in ([0, 1, 2, 2], [0, 1, 2, 4], [0, 1, 2, -1], [3, 3, 3, 3]):  # B = 4 entries each
        assert decode_call(lib, order=bad) == pa.PA_ERR_INVALID_ARG, bad
    pp = lib.pa_decode_partition_tokens() // 16
    big = np.arange(1025, dtype=np.int32)
    assert decode_call(lib, B=1025, order=big) == pa.PA_ERR_INVALID_ARG
    # 512 sequences of 3 partitions each: 1536 items
    assert decode_call(lib, B=512, mb=2 * pp + 1, order=np.arange(512)) == pa.PA_ERR_INVALID_ARG
    # 65 partitions of one sequence
    assert decode_call(lib, B=1, mb=64 * pp + 1, order=[0]) == pa.PA_ERR_INVALID_ARG
    # the order is checked before the rest: a valid one leaves the other errors as they were
    assert decode_call(lib, ps=32, order=[3, 2, 1, 0]) == pa.PA_ERR_UNSUPPORTED
    assert decode_call(lib, q=0, order=[3, 2, 1, 0]) == pa.PA_ERR_INVALID_ARG
    assert decode_call(lib, B=0, q=0, out=0, order=[]) == pa.PA_OK


def test_device_order_validation(pa):
    """A device order is not checked on the host beyond its pointer: it may not come with a host
    order, and it must be 16-byte aligned; with any number of sequences and partitions it is
    otherwise accepted (the fake pointers below fail later checks, so nothing is launched)."""
    lib = pa.lib()
    assert decode_call(lib, order=[0, 1, 2, 3], dorder=FAKE) == pa.PA_ERR_INVALID_ARG
    assert decode_call(lib, q=0, dorder=FAKE + 4) == pa.PA_ERR_INVALID_ARG
    assert decode_call(lib, ps=32, dorder=FAKE) == pa.PA_ERR_UNSUPPORTED  # the order passes, the page size fails
    pp = lib.pa_decode_partition_tokens() // 16
    need = lib.pa_decode_workspace_bytes(2000, 70 * pp)
    assert decode_call(lib, B=2000, mb=70 * pp, dorder=FAKE) == pa.PA_ERR_WORKSPACE  # no 1024-item bound
    assert decode_call(lib, B=2000, mb=70 * pp, dorder=FAKE, ws=FAKE, wsb=need, q=0) == pa.PA_ERR_INVALID_ARG
    assert decode_call(lib, B=0, q=0, out=0, dorder=FAKE) == pa.PA_OK


def test_order_by_length_validation(pa):
    """pa_order_by_length refuses, before launching anything, a batch beyond PA_MAX_DISPATCH_ORDER,
    max_blocks < 1, runs outside [1, 64] (long) or [0, 64] (short), NULL or misaligned arrays and
    overlapping arrays; an empty batch is a no-op."""
    lib = pa.lib()
    v = ctypes.c_void_p
    F = FAKE

    def call(lens=F, n=4, mb=8, order=F + 4096, k=1, m=0):
        return lib.pa_order_by_length(v(lens) if lens else None, n, mb, k, m, v(order) if order else None, None)

    assert call(n=-1) == pa.PA_ERR_INVALID_ARG
    for k, m in ((0, 0), (-1, 1), (65, 0), (1, -1), (1, 65)):
        assert call(k=k, m=m) == pa.PA_ERR_INVALID_ARG, (k, m)
        assert call(k=k, m=m, n=0, lens=0, order=0) == pa.PA_ERR_INVALID_ARG, (k, m)
    assert call(n=1025) == pa.PA_ERR_INVALID_ARG
    assert call(mb=0) == pa.PA_ERR_INVALID_ARG
    assert call(lens=0) == pa.PA_ERR_INVALID_ARG
    assert call(order=0) == pa.PA_ERR_INVALID_ARG
    assert call(lens=F + 4) == pa.PA_ERR_INVALID_ARG
    assert call(order=F + 8) == pa.PA_ERR_INVALID_ARG
    assert call(order=F) == pa.PA_ERR_INVALID_ARG            # the same array
    assert call(order=F + 16, n=5) == pa.PA_ERR_INVALID_ARG  # 20 bytes each: they overlap
    assert call(n=0, lens=0, order=0) == pa.PA_OK


def test_dispatch_order_helper(pa):
    """The longest-first helper is a stable descending sort of the lengths."""
    rng = np.random.default_rng(5)
    for n in (0, 1, 7, 256, 1000):
        lens = rng.integers(1, 40, size=n).astype(np.int32)  # many ties
        got = pa.dispatch_order_longest_first(lens)
        assert np.array_equal(got, np.argsort(-lens.astype(np.int64), kind="stable").astype(np.int32))
    assert pa.lib().pa_dispatch_order_longest_first(None, 3, None) == pa.PA_ERR_INVALID_ARG
    assert pa.lib().pa_dispatch_order_longest_first(None, -1, None) == pa.PA_ERR_INVALID_ARG
    assert pa.lib().pa_dispatch_order_longest_first(None, 0, None) == pa.PA_OK


def test_workspace_arithmetic(pa):
    lib = pa.lib()
    pt = lib.pa_decode_partition_tokens()
    assert pt % 16 == 0 and pt >= 16
    pp = pt // 16
    for B, mb in [(1, 1), (3, pp), (3, pp + 1), (64, 128), (256, 128), (7, 1000)]:
        parts = -(-mb // pp)
        expect = 0 if parts <= 1 else B * 32 * parts * 66 * 4
        assert lib.pa_decode_workspace_bytes(B, mb) == expect
    assert lib.pa_decode_workspace_bytes(0, 128) == 0
    assert lib.pa_decode_workspace_bytes(5, 0) == 0


def test_append_and_prefill_validation(pa):
    lib = pa.lib()
    v = ctypes.c_void_p
    F = v(FAKE)

    def app(q=F, kn=F, vn=F, kp=F, vp=F, bt=F, cl=F, rope=F, B=2, mb=4, P=16, ps=16, mp=64):
        return lib.pa_append_kv_rope(q, kn, vn, kp, vp, bt, cl, rope, B, mb, P, ps, mp, None, None)

    assert app(ps=8) == pa.PA_ERR_UNSUPPORTED
    assert app(B=-2) == pa.PA_ERR_INVALID_ARG
    assert app(mp=0) == pa.PA_ERR_INVALID_ARG
    assert app(kn=None) == pa.PA_ERR_INVALID_ARG
    assert app(rope=v(FAKE + 4)) == pa.PA_ERR_INVALID_ARG
    assert app(q=v(FAKE + 2)) == pa.PA_ERR_INVALID_ARG
    assert app(B=0) == pa.PA_OK

    def pre(B=2, C=8, ps=16, odt=0, q=F, mp=64):
        return lib.pa_prefill_chunk(F, q, F, F, F, F, F, F, F, B, C, 4, 16, ps, mp, 0.125, odt, None, None)

    assert pre(ps=32) == pa.PA_ERR_UNSUPPORTED
    assert pre(C=-1) == pa.PA_ERR_INVALID_ARG
    assert pre(mp=0) == pa.PA_ERR_INVALID_ARG


def test_i8_validation(pa):
    lib = pa.lib()
    v = ctypes.c_void_p
    F = v(FAKE)
    assert lib.pa_i8_pool_bytes(10) == 10 * 8 * 2176
    assert lib.pa_i8_pool_bytes(0) == 0

    def quant(pool=F, kp=F, vp=F, ids=F, n=4, P=16):
        return lib.pa_quantize_pages_i8(pool, kp, vp, ids, n, P, None, None)

    assert quant(n=-1) == pa.PA_ERR_INVALID_ARG
    assert quant(P=0) == pa.PA_ERR_INVALID_ARG
    assert quant(ids=None, n=17) == pa.PA_ERR_INVALID_ARG   # more pages than the pool holds
    assert quant(pool=None) == pa.PA_ERR_INVALID_ARG
    assert quant(kp=v(FAKE + 8)) == pa.PA_ERR_INVALID_ARG
    assert quant(n=0, pool=None) == pa.PA_OK

    def app(q=F, pool=F, B=2, ps=16, mp=64, kn=F):
        return lib.pa_append_kv_rope_i8(q, kn, F, pool, F, F, F, B, 4, 16, ps, mp, None, None)

    assert app(ps=8) == pa.PA_ERR_UNSUPPORTED
    assert app(mp=0) == pa.PA_ERR_INVALID_ARG
    assert app(pool=None) == pa.PA_ERR_INVALID_ARG
    assert app(kn=v(FAKE + 2)) == pa.PA_ERR_INVALID_ARG
    assert app(B=0) == pa.PA_OK

    def dec(out=F, pool=F, B=4, mb=8, ps=16, odt=0, scale=0.125, ws=None, wsb=0):
        return lib.pa_decode_gqa_i8(out, F, pool, F, F, B, mb, 64, ps, scale, odt, ws, wsb, None, None, None, None)

    assert dec(ps=32) == pa.PA_ERR_UNSUPPORTED
    assert dec(odt=3) == pa.PA_ERR_UNSUPPORTED
    assert dec(pool=None) == pa.PA_ERR_INVALID_ARG
    assert dec(out=v(FAKE + 4)) == pa.PA_ERR_INVALID_ARG
    assert dec(scale=float("inf")) == pa.PA_ERR_INVALID_ARG
    assert dec(B=0, out=None) == pa.PA_OK
    need = lib.pa_decode_workspace_bytes(4, 1000)
    assert need > 0 and dec(mb=1000) == pa.PA_ERR_WORKSPACE

    def pre8(B=2, C=8, ps=16, odt=0, q=F, pool=F, mp=64, mb=4):
        return lib.pa_prefill_chunk_i8(F, q, F, F, pool, F, F, F, B, C, mb, 16, ps, mp, 0.125, odt, None, None)

    assert pre8(ps=32) == pa.PA_ERR_UNSUPPORTED
    assert pre8(odt=5) == pa.PA_ERR_UNSUPPORTED
    assert pre8(mb=513) == pa.PA_ERR_UNSUPPORTED
    assert pre8(C=-1) == pa.PA_ERR_INVALID_ARG
    assert pre8(mp=0) == pa.PA_ERR_INVALID_ARG
    assert pre8(pool=None) == pa.PA_ERR_INVALID_ARG
    assert pre8(q=v(FAKE + 8)) == pa.PA_ERR_INVALID_ARG
    assert pre8(B=0, q=None, pool=None) == pa.PA_OK
    assert pre8(C=0, q=None, pool=None) == pa.PA_OK

    def fused(rope=F, mp=64):
        return lib.pa_append_decode_gqa_i8(F, F, F, F, F, F, F, rope, 4, 8, 64, 16, mp, 0.125, 0, None, 0, None,
                                           None, None, None)

    assert fused(rope=None) == pa.PA_ERR_INVALID_ARG
    assert fused(mp=0) == pa.PA_ERR_INVALID_ARG


def test_argmax_validation(pa):
    lib = pa.lib()
    v = ctypes.c_void_p
    F = v(FAKE)
    chunk_bf16, chunk_fp32 = 256 * 8 * 8, 256 * 8 * 4
    assert -(-128256 // chunk_bf16) > 1 and -(-128256 // chunk_fp32) > 1
    assert lib.pa_argmax_workspace_bytes(64, 128256, 0) == 64 * 16      # per row: running key + arrival count
    assert lib.pa_argmax_workspace_bytes(64, 128256, 1) == 64 * 16
    assert lib.pa_argmax_workspace_bytes(5, chunk_bf16, 0) == 0          # one chunk per row: no workspace
    assert lib.pa_argmax_workspace_bytes(5, 100, 2) == 0

    def am(out=F, lg=F, rows=4, vocab=128256, dt=0, ws=None, wsb=0):
        return lib.pa_argmax(out, lg, rows, vocab, dt, ws, wsb, None)

    assert am(dt=2) == pa.PA_ERR_UNSUPPORTED
    assert am(vocab=0) == pa.PA_ERR_INVALID_ARG
    assert am(rows=-1) == pa.PA_ERR_INVALID_ARG
    assert am(out=None) == pa.PA_ERR_INVALID_ARG
    assert am(lg=v(FAKE + 1)) == pa.PA_ERR_INVALID_ARG
    assert am(dt=1, lg=v(FAKE + 2)) == pa.PA_ERR_INVALID_ARG
    assert am() == pa.PA_ERR_WORKSPACE
    need = lib.pa_argmax_workspace_bytes(4, 128256, 0)
    assert am(ws=F, wsb=need - 8) == pa.PA_ERR_WORKSPACE
    assert am(ws=v(FAKE + 4), wsb=need) == pa.PA_ERR_WORKSPACE
    assert am(rows=0, out=None) == pa.PA_OK


def test_stream_read_probe_validation(pa):
    lib = pa.lib()
    v = ctypes.c_void_p
    F = v(FAKE)
    assert lib.pa_probe_stream_read(F, 1 << 20, None, None) == pa.PA_ERR_INVALID_ARG
    assert lib.pa_probe_stream_read(None, 1 << 20, F, None) == pa.PA_ERR_INVALID_ARG
    assert lib.pa_probe_stream_read(v(FAKE + 8), 1 << 20, F, None) == pa.PA_ERR_INVALID_ARG
    assert lib.pa_probe_stream_read(F, (1 << 20) + 8, F, None) == pa.PA_ERR_INVALID_ARG
    assert lib.pa_probe_stream_read(F, 1 << 20, v(FAKE + 2), None) == pa.PA_ERR_INVALID_ARG
    assert lib.pa_probe_stream_read(None, 0, None, None) == pa.PA_OK


def test_rope_table_fill(pa):
    """The table holds the C library's double cos / sin of pos * pow(theta, -2i/64) exactly
    (Python's math module calls the same libm)."""
    t = np.empty((300, 32, 2), np.float64)
    assert pa.lib().pa_rope_table_fill_host(t.ctypes.data_as(ctypes.c_void_p), 300, 500000.0) == 0
    for pos in range(300):
        for i in range(32):
            a = float(pos) * math.pow(500000.0, -(2.0 * i) / 64.0)
            assert t[pos, i, 0] == math.cos(a) and t[pos, i, 1] == math.sin(a), (pos, i)
    assert pa.lib().pa_rope_table_fill_host(None, 3, 500000.0) == pa.PA_ERR_INVALID_ARG
    assert pa.lib().pa_rope_table_fill_host(t.ctypes.data_as(ctypes.c_void_p), 0, 500000.0) == pa.PA_ERR_INVALID_ARG


def test_abi_version_matches_header():
    from paged_kv_gqa_append_amd import binding

    hdr = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "pa.h")).read()
    assert int(re.search(r"#define PA_ABI_VERSION (\d+)", hdr).group(1)) == binding.ABI_VERSION
    binding._require_abi(binding.ABI_VERSION)
    with pytest.raises(RuntimeError, match="rebuild"):
        binding._require_abi(binding.ABI_VERSION - 1)


def test_binding_refuses_without_library(tmp_path, monkeypatch):
    from paged_kv_gqa_append_amd import binding

    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding, "_LIB_PATH", str(tmp_path / "libpa.so"))
    with pytest.raises(RuntimeError, match="no fallback"):
        binding.lib()


def test_device_error_readback_validation(pa):
    """pa_get_device_error refuses a NULL or misaligned flag word before touching the runtime."""
    lib = pa.lib()
    assert lib.pa_get_device_error(None, 0, None) == -pa.PA_ERR_INVALID_ARG
    assert lib.pa_get_device_error(ctypes.c_void_p(FAKE + 2), 1, None) == -pa.PA_ERR_INVALID_ARG


def test_build_id_matches_tree(pa):
    """The library in the tree was built from the sources in the tree: its embedded build id
    (read through the ABI and from the file) is the digest of today's sources and flags."""
    from paged_kv_gqa_append_amd import build

    got = pa.lib().pa_build_id().decode()
    assert re.fullmatch(r"[0-9a-f]{64}", got)
    assert got == build.source_digest() == build.built_digest()
    assert build.is_current()


def test_stale_library_is_refused(pa, monkeypatch):
    """A build id that differs from the sources' digest makes the binding refuse the library."""
    from paged_kv_gqa_append_amd import binding

    binding._require_current(__import__("paged_kv_gqa_append_amd.build", fromlist=["x"]).source_digest())
    with pytest.raises(RuntimeError, match="rebuild"):
        binding._require_current("0" * 64)


def test_digest_tracks_sources(tmp_path, monkeypatch):
    """The digest covers the kernel sources, their headers and the ABI header: a copy of the tree
    hashes the same, and a one-byte change to any of those files changes it."""
    import shutil

    from paged_kv_gqa_append_amd import build

    base = build.source_digest()
    rel = [os.path.relpath(f, build.ROOT) for f in build.digest_inputs()]
    assert "include/pa.h" in rel and any(r.endswith(".h") and "csrc" in r for r in rel)
    root = tmp_path / "tree"
    shutil.copytree(os.path.join(build.ROOT, "paged_kv_gqa_append_amd", "csrc"),
                    root / "paged_kv_gqa_append_amd" / "csrc")
    shutil.copytree(os.path.join(build.ROOT, "include"), root / "include")
    monkeypatch.setattr(build, "ROOT", str(root))
    monkeypatch.setattr(build, "CSRC", str(root / "paged_kv_gqa_append_amd" / "csrc"))
    monkeypatch.setattr(build, "INCLUDE", str(root / "include"))
    assert build.source_digest() == base
    for r in (rel[0], "paged_kv_gqa_append_amd/csrc/pa_decode_core.h", "include/pa.h"):
        f = root / r
        data = f.read_bytes()
        f.write_bytes(data + b"\n")
        assert build.source_digest() != base, r
        f.write_bytes(data)
    assert build.source_digest() == base


def test_dispatch_order_length_refused(pa):
    """The library reads exactly num_seqs order entries through a bare pointer, so the binding
    refuses a shorter or longer array before calling it (host tensors: nothing is launched)."""
    import torch

    B, mb, P = 3, 2, 8
    kp = torch.zeros((P, 8, 16, 64), dtype=torch.bfloat16)
    q = torch.zeros((B, 32, 64), dtype=torch.bfloat16)
    out = torch.zeros((B, 32, 64), dtype=torch.bfloat16)
    bt = torch.zeros((B, mb), dtype=torch.int32)
    lens = torch.ones(B, dtype=torch.int32)
    kn = torch.zeros((B, 8, 64), dtype=torch.bfloat16)
    table = torch.zeros((64, 32, 2), dtype=torch.float64)
    i8 = torch.zeros((P, 8, 2176), dtype=torch.uint8)
    for bad in ([1, 0], [2, 1, 0, 3], [[0, 1, 2]]):
        with pytest.raises(ValueError, match="exactly num_seqs"):
            pa.decode_gqa(out, q, kp, kp, bt, lens, dispatch_order=bad)
        with pytest.raises(ValueError, match="exactly num_seqs"):
            pa.append_decode_gqa(out, q, kn, kn, kp, kp, bt, lens, table, dispatch_order=bad)
        with pytest.raises(ValueError, match="exactly num_seqs"):
            pa.decode_gqa_i8(out, q, i8, bt, lens, dispatch_order=bad)
        with pytest.raises(ValueError, match="exactly num_seqs"):
            pa.append_decode_gqa_i8(out, q, kn, kn, i8, bt, lens, table, dispatch_order=bad)
    arr, ptr, dptr = pa._order(np.array([2, 0, 1], np.int32), B)
    assert arr.shape == (3,) and ptr.value == arr.ctypes.data and dptr is None
    # a tensor is a device order: int32 of exactly num_seqs entries on the call's device
    t = torch.tensor([2, 0, 1], dtype=torch.int32)
    keep, ptr, dptr = pa._order(t, B, t.device)
    assert keep is t and ptr is None and dptr.value == t.data_ptr()
    for bad in (torch.tensor([1, 0], dtype=torch.int32), torch.tensor([2, 0, 1], dtype=torch.int64)):
        with pytest.raises((ValueError, TypeError)):
            pa.decode_gqa(out, q, kp, kp, bt, lens, dispatch_order=bad)


def test_noalloc_size_limit(pa):
    """pa_append_decode_gqa_noalloc refuses a batch whose partials exceed its scratch before
    anything else happens (the fake pointers are never touched), and validates arguments like
    pa_append_decode_gqa when no scratch is needed."""
    lib = pa.lib()
    v = ctypes.c_void_p
    F = v(FAKE)
    pp = lib.pa_decode_partition_tokens() // 16

    def na(B=4, mb=8, ps=16, mp=64, q=F, rope=F):
        return lib.pa_append_decode_gqa_noalloc(F, q, F, F, F, F, F, F, rope, B, mb, 64, ps, mp, 0.125, 0, None,
                                                None, None, None)

    assert lib.pa_decode_workspace_bytes(64, 16 * pp + 1) > pa.NOALLOC_SCRATCH_BYTES
    assert na(B=64, mb=16 * pp + 1) == pa.PA_ERR_WORKSPACE
    assert lib.pa_decode_workspace_bytes(64, 15 * pp) <= pa.NOALLOC_SCRATCH_BYTES
    assert na(ps=32) == pa.PA_ERR_UNSUPPORTED
    assert na(mp=0) == pa.PA_ERR_INVALID_ARG
    assert na(q=None) == pa.PA_ERR_INVALID_ARG
    assert na(rope=None) == pa.PA_ERR_INVALID_ARG
    assert na(B=0) == pa.PA_OK
    m = re.search(r"#define PA_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", open(HEADER).read())
    assert int(m.group(1)) << int(m.group(2)) == pa.NOALLOC_SCRATCH_BYTES
