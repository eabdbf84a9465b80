"""GPU parity of the INT8 K/V page calls against the fp64 oracle.

* pa_quantize_pages_i8: every byte of the INT8 pool equals the oracle's
  quantisation of the same bf16 pages (codes and scales are integer/binary32
  decisions taken in binary32 on both sides), unlisted pages untouched.
* pa_append_kv_rope_i8: the whole pool (the appended slots' K/V codes and
  scales included) and the rotated q bit for bit: the device rotates with the
  oracle's fp64 operations, so the rotated bf16 K row it quantises is the
  oracle's.
* pa_decode_gqa_i8 / pa_append_decode_gqa_i8: outputs within the stated
  tolerance of the oracle's decode over the same INT8 pool (bf16 out
  1e-2 + 1e-2|ref|, fp32 out 2e-3 + 2e-3|ref|); the fused call is bitwise the
  two separate calls; contexts past one partition; unused slots hold NaN scales
  and random codes.
* Full size: the batch-64 x 2048 and ragged batch-256 workloads' pools
  quantised on the device are bit-identical, on whole layers' pages, to the
  oracle's quantisation of the same bf16 pages (copied to the host before any
  of our kernels ran); the fused append + decode matches the oracle on every
  sequence of those layers, and the pool after the append bit for bit.
The INT8 pools the oracle reads are built on the host by the oracle itself.
"""
import numpy as np
import pytest
import torch

import oracle
from _gpu_helpers import (TOL_BF16, TOL_FP32, assert_close, assert_rope_equal, dev, rope, to_dev_bf16, to_dev_i32,
                          to_host_bits, to_host_f64)
from _gpu_helpers import guarded_empty, guarded_full, guarded_flags, to_dev_u8, guarded_workspace, guarded_pool
from paged_kv_gqa_append_amd import binding
from paged_kv_gqa_append_amd import workloads as W

pytestmark = pytest.mark.gpu

TILE = 2176
NAN32 = np.array([0x7FC00000], np.uint32).view(np.uint8)


def k_pos(t, d):
    """Byte of K element d of slot t in a 2176-byte tile (include/pa.h)."""
    return (((d % 32) // 8) * 16 + t) * 16 + (d // 32) * 8 + d % 8


def v_pos(t, d):
    """Byte of V element d of slot t in a tile (include/pa.h)."""
    return 1024 + ((t // 4) * 16 + d % 16) * 16 + (d // 16) * 4 + t % 4


K_BYTES = np.array([[k_pos(t, d) for d in range(64)] for t in range(16)])  # [16][64]
V_BYTES = np.array([[v_pos(t, d) for d in range(64)] for t in range(16)])
K_SCALE = [2048 + 4 * t for t in range(16)]
V_SCALE = [2112 + 4 * t for t in range(16)]


def poison_i8(pool, block_tables, lens, seed):
    """Every slot no sequence uses (any layer): NaN scales and random codes."""
    rng = np.random.default_rng(seed)
    used = np.zeros((pool.shape[0], 16), bool)
    for layer in range(block_tables.shape[0]):
        p, t = W.used_slots(block_tables[layer], lens)
        used[p, t] = True
    for p, t in np.argwhere(~used):
        page = pool[p]  # [8][2176] view
        for idx in (K_BYTES[t], V_BYTES[t]):
            page[:, idx] = rng.integers(0, 256, (8, 64), dtype=np.uint8)
        page[:, K_SCALE[t]:K_SCALE[t] + 4] = NAN32
        page[:, V_SCALE[t]:V_SCALE[t] + 4] = NAN32


def host_i8(case, poison=True):
    pool = oracle.quantize_pages_i8(case.k_pool, case.v_pool)
    if poison:
        poison_i8(pool, case.block_tables, case.context_lens, case.seed + 1000)
    return pool


def oracle_decode_i8(case, pool, q_bits=None):
    out, rc = oracle.decode_gqa_i8(case.q[0] if q_bits is None else q_bits, pool, case.block_tables[0],
                                   case.context_lens, case.num_pages, case.scale)
    assert rc == oracle.OK
    return out


EDGE = [1, 2, 15, 16, 17, 31, 33, 255, 256, 257, 511, 512, 513, 1023, 1024, 1025, 2047, 2048]
CASES = {
    "tiny": lambda: W.tiny_decode(),
    "batch8": lambda: W.batch8_decode(),
    "edges": lambda: W.make_decode_case("edges", 71, EDGE, dist="normal", max_blocks=130),
    "ragged_outliers": lambda: W.make_decode_case("ragged", 72, W.ragged_lengths(72, 24), dist="normal",
                                                  layout="fragmented", outlier_frac=0.01, max_blocks=128),
    "long": lambda: W.make_decode_case("long", 73, [1, 17, 2048, 2049, 3000, 4113], dist="normal", max_blocks=260),
}


def test_quantize_pages_bitexact():
    case = W.make_decode_case("quant", 74, [700, 1, 33, 2048], dist="normal", poison=False, outlier_frac=0.02)
    kp, vp = case.k_pool.copy(), case.v_pool.copy()
    kp[0, 2, 5, :] = 0                                                  # an all-zero row: scale 0, codes 0
    vp[1, 0, 3, :] = W.f32_to_bf16_bits(np.full(64, 1e-30, np.float32))  # tiny values
    P = case.num_pages
    rng = np.random.default_rng(75)
    start = rng.integers(0, 256, (P, 8, TILE), dtype=np.uint8)
    ids = np.sort(rng.choice(P, size=P // 2, replace=False)).astype(np.int32)
    full = oracle.quantize_pages_i8(kp, vp)
    print(f"quantize pages P={P} listed={len(ids)}", flush=True)
    # listed pages only
    pool = to_dev_u8(start)
    flags = guarded_flags()
    binding.quantize_pages_i8(pool, to_dev_bf16(kp), to_dev_bf16(vp), to_dev_i32(ids), device_flags=flags)
    torch.cuda.synchronize()
    want = start.copy()
    want[ids] = full[ids]
    assert np.array_equal(pool.cpu().numpy(), want)
    assert int(flags.item()) == 0
    # all pages
    pool = to_dev_u8(start)
    binding.quantize_pages_i8(pool, to_dev_bf16(kp), to_dev_bf16(vp))
    torch.cuda.synchronize()
    assert np.array_equal(pool.cpu().numpy(), full)
    # an id outside the pool is skipped and flagged
    bad = np.array([0, P, 3, -1], np.int32)
    pool = to_dev_u8(start)
    binding.quantize_pages_i8(pool, to_dev_bf16(kp), to_dev_bf16(vp), to_dev_i32(bad), device_flags=flags)
    torch.cuda.synchronize()
    want = start.copy()
    want[[0, 3]] = full[[0, 3]]
    assert np.array_equal(pool.cpu().numpy(), want)
    assert int(flags.item()) & binding.PA_DEVERR_PAGE_ID


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_decode_i8_parity(name, out_dtype):
    case = CASES[name]()
    print(f"i8 decode parity case={name} B={case.num_seqs} out={out_dtype}", flush=True)
    pool = host_i8(case)
    out = guarded_empty((case.num_seqs, 32, 64), out_dtype)
    flags = guarded_flags()
    binding.decode_gqa_i8(out, to_dev_bf16(case.q[0]), to_dev_u8(pool), to_dev_i32(case.block_tables[0]),
                          to_dev_i32(case.context_lens), case.scale,
                          workspace=guarded_workspace(case.num_seqs, case.max_blocks),
                          device_flags=flags)
    torch.cuda.synchronize()
    got = to_host_f64(out)
    assert_close(got, oracle_decode_i8(case, pool), TOL_BF16 if out_dtype == torch.bfloat16 else TOL_FP32, name)
    assert int(flags.item()) == 0


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_decode_i8_very_long_contexts(out_dtype):
    """Contexts up to 32,768 tokens over INT8 pages: 16 partitions of 128 pages and their merge,
    2,048-entry block-table rows."""
    case = W.make_decode_case("very_long", 75, [32768, 20001, 1, 4097], dist="normal", max_blocks=2048)
    pool = host_i8(case)
    out = guarded_empty((case.num_seqs, 32, 64), out_dtype)
    flags = guarded_flags()
    binding.decode_gqa_i8(out, to_dev_bf16(case.q[0]), to_dev_u8(pool), to_dev_i32(case.block_tables[0]),
                          to_dev_i32(case.context_lens), case.scale,
                          workspace=guarded_workspace(case.num_seqs, case.max_blocks), device_flags=flags)
    torch.cuda.synchronize()
    assert int(flags.item()) == 0
    assert_close(to_host_f64(out), oracle_decode_i8(case, pool), TOL_BF16 if out_dtype == torch.bfloat16 else TOL_FP32,
                 "very long")


WIDE_V = {
    # |v| up to 1e6 (the plain f16 form of the weights overflowed past about 3.2e4), with rows of
    # 1e-6: every output within the stated tolerance
    "edge": ([1.0, 1.0, 4.0e4, 1.0e6, 1.0e-6], [.5, .2, .15, .1, .05]),
    # rows of 1e30 beside rows of 1e5 and of 1e-6 in one head: within the tolerance plus 2^-16 of
    # the head's largest |V| (the weights reach the f16 MFMA through one exponent per wave, so rows
    # about 2^30 below the largest lose their precision first)
    "extreme": ([1.0, 1.0, 4.0e4, 1.0e6, 1.0e-6, 1.0e30], [.5, .2, .1, .1, .08, .02]),
}


@pytest.mark.parametrize("name", list(WIDE_V))
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_decode_i8_wide_v_range(name, out_dtype):
    """V rows far beyond what an f16 weight times a V scale can hold without an exponent
    offset, mixed with ordinary rows and rows of 1e-6 in the same pages and sequences, some
    past one partition, against the oracle over the same INT8 pool.
    The enlarged rows are one-signed (|v| x factor): with random signs, large terms can cancel
    to outputs a million times smaller, and then any fp32 accumulation (bf16 pools included)
    misses a bar relative to the output; that is the sum's conditioning, not the range this
    test is about."""
    factors, probs = WIDE_V[name]
    lens = [40, 600, 2048, 17, 2500]
    case = W.make_decode_case("wide_v", 76, lens, dist="normal", max_blocks=160, poison=False)
    rng = np.random.default_rng(77)
    rows = W.bf16_bits_to_f32(case.v_pool).astype(np.float64)  # [P][8][16][64]
    factor = rng.choice(factors, size=rows.shape[:3], p=probs)
    big = (factor > 1.0)[..., None]
    vp = W.f32_to_bf16_bits((np.where(big, np.abs(rows), rows) * factor[..., None]).astype(np.float32))
    case.v_pool = vp
    vmag = np.abs(W.bf16_bits_to_f32(vp).astype(np.float64)).max(axis=3)  # [P][8][16] row max |v|
    print(f"i8 wide V range {name} B={case.num_seqs} out={out_dtype} max|v|={vmag.max():.3g}", flush=True)
    pool = host_i8(case)
    out = guarded_empty((case.num_seqs, 32, 64), out_dtype)
    flags = guarded_flags()
    binding.decode_gqa_i8(out, to_dev_bf16(case.q[0]), to_dev_u8(pool), to_dev_i32(case.block_tables[0]),
                          to_dev_i32(case.context_lens), case.scale,
                          workspace=guarded_workspace(case.num_seqs, case.max_blocks), device_flags=flags)
    torch.cuda.synchronize()
    ref = oracle_decode_i8(case, pool)
    got = to_host_f64(out)
    tol = TOL_BF16 if out_dtype == torch.bfloat16 else TOL_FP32
    assert int(flags.item()) == 0
    if name == "edge":
        assert np.abs(ref).max() > 1e4  # the large rows do reach the outputs
        assert_close(got, ref, tol, "wide V range (edge)")
        return
    # the largest |V| each (sequence, KV head) attends, broadcast over its 4 q heads and 64 dims
    head_max = np.zeros((case.num_seqs, 8))
    for s, L in enumerate(case.context_lens):
        t = np.arange(int(L))
        pg = case.block_tables[0][s, t // 16]
        head_max[s] = vmag[pg, :, t % 16].max(axis=0)
    extra = 2.0 ** -16 * np.repeat(head_max, 4, axis=1)[:, :, None]
    assert np.abs(ref).max() > 1e20
    assert np.all(np.isfinite(got))
    err = np.abs(got - ref)
    bad = err > tol[0] + tol[1] * np.abs(ref) + extra
    assert not bad.any(), f"{int(bad.sum())} outputs outside tolerance + 2^-16 of the head's largest |V|"


def read_row(pool, page, head, t, which):
    codes = pool[page, head, (K_BYTES if which == "k" else V_BYTES)[t]].view(np.int8)
    s = (K_SCALE if which == "k" else V_SCALE)[t]
    sc = pool[page, head, s:s + 4].view(np.float32)[0]
    return codes, sc


def test_append_i8_against_oracle():
    case = W.batch8_decode()
    pool = host_i8(case)
    table = rope()
    q = to_dev_bf16(case.q[0])
    dpool = to_dev_u8(pool)
    flags = guarded_flags()
    binding.append_kv_rope_i8(q, to_dev_bf16(case.k_new[0]), to_dev_bf16(case.v_new[0]), dpool,
                              to_dev_i32(case.block_tables[0]), to_dev_i32(case.context_lens), table,
                              device_flags=flags)
    torch.cuda.synchronize()
    assert int(flags.item()) == 0
    got = dpool.cpu().numpy()
    ref = pool.copy()
    oq = case.q[0].copy()
    assert oracle.append_kv_rope_i8(oq, case.k_new[0], case.v_new[0], ref, case.block_tables[0], case.context_lens,
                                    case.num_pages, case.theta) == oracle.OK
    # the whole pool, codes and scales, bit for bit (the rotation is the oracle's)
    diff = got != ref
    assert not diff.any(), f"{int(diff.sum())} pool bytes differ from the oracle"
    assert_rope_equal(to_host_bits(q), oq, "rotated q")


@pytest.mark.parametrize("name", ["tiny", "edges", "long"])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_fused_i8_equals_separate(name, out_dtype):
    case = CASES[name]()
    if name == "tiny":
        case.context_lens[:] = 64
    print(f"i8 fused vs separate case={name} out={out_dtype}", flush=True)
    pool = host_i8(case)
    table = rope(4200)
    bt, lens = to_dev_i32(case.block_tables[0]), to_dev_i32(case.context_lens)
    kn, vn = to_dev_bf16(case.k_new[0]), to_dev_bf16(case.v_new[0])
    ws = guarded_workspace(case.num_seqs, case.max_blocks)
    # separate
    q1, p1 = to_dev_bf16(case.q[0]), to_dev_u8(pool)
    o1 = guarded_empty((case.num_seqs, 32, 64), out_dtype)
    binding.append_kv_rope_i8(q1, kn, vn, p1, bt, lens, table)
    binding.decode_gqa_i8(o1, q1, p1, bt, lens, case.scale, workspace=ws)
    # fused
    q2, p2 = to_dev_bf16(case.q[0]), to_dev_u8(pool)
    o2 = guarded_empty((case.num_seqs, 32, 64), out_dtype)
    binding.append_decode_gqa_i8(o2, q2, kn, vn, p2, bt, lens, table, case.scale, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16 if out_dtype == torch.bfloat16 else torch.int32),
                       o2.view(torch.int16 if out_dtype == torch.bfloat16 else torch.int32))
    assert torch.equal(q1.view(torch.int16), q2.view(torch.int16))
    assert torch.equal(p1, p2)
    # and against the oracle's append + decode
    ref_pool, oq = pool.copy(), case.q[0].copy()
    assert oracle.append_kv_rope_i8(oq, case.k_new[0], case.v_new[0], ref_pool, case.block_tables[0],
                                    case.context_lens, case.num_pages, case.theta) == oracle.OK
    ref, rc = oracle.decode_gqa_i8(oq, ref_pool, case.block_tables[0], case.context_lens, case.num_pages, case.scale)
    assert rc == oracle.OK
    assert_close(to_host_f64(o2), ref, TOL_BF16 if out_dtype == torch.bfloat16 else TOL_FP32, name)
    # out may alias q
    q3, p3 = to_dev_bf16(case.q[0]), to_dev_u8(pool)
    binding.append_decode_gqa_i8(q3, q3, kn, vn, p3, bt, lens, table, case.scale, workspace=ws)
    torch.cuda.synchronize()
    if out_dtype == torch.bfloat16:
        assert torch.equal(q3.view(torch.int16), o1.view(torch.int16))
    assert torch.equal(p3, p1)


def test_single_token_returns_its_v():
    """L = 1: the weight is exactly 1, so out = V scale x code up to the fp32
    roundings of the offset encoding: the MFMA accumulates (1152 + code) x
    scale and the correction subtracts 1152 x scale, each within 2^-24 of a
    value below 1280 x scale, so |out - code x scale| < 2^-12 x scale."""
    case = W.make_decode_case("one", 76, [1] * 5, dist="normal")
    pool = host_i8(case)
    out = guarded_empty((5, 32, 64), torch.float32)
    binding.decode_gqa_i8(out, to_dev_bf16(case.q[0]), to_dev_u8(pool), to_dev_i32(case.block_tables[0]),
                          to_dev_i32(case.context_lens), case.scale)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    for s in range(5):
        pg = case.block_tables[0][s, 0]
        for h in range(32):
            codes, sc = read_row(pool, pg, h // 4, 0, "v")
            want = codes.astype(np.float64) * float(sc)
            assert np.all(np.abs(got[s, h] - want) <= float(sc) * 2.0 ** -12)


def test_i8_device_errors():
    case = W.make_decode_case("err", 77, [40, 40, 40], dist="normal", max_blocks=4)
    pool = host_i8(case)
    bt = case.block_tables[0].copy()
    lens = case.context_lens.copy()
    lens[0] = 0                 # bad length
    bt[1, 1] = case.num_pages   # bad page id in the used range
    out = guarded_full((3, 32, 64), 7.0, torch.float32)
    flags = guarded_flags()
    binding.decode_gqa_i8(out, to_dev_bf16(case.q[0]), to_dev_u8(pool), to_dev_i32(bt), to_dev_i32(lens),
                          case.scale, device_flags=flags)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.all(got[0] == 0) and np.all(got[1] == 0)
    assert int(flags.item()) == binding.PA_DEVERR_CONTEXT_LEN | binding.PA_DEVERR_PAGE_ID
    ok = case.context_lens[2:]
    ref, rc = oracle.decode_gqa_i8(case.q[0][2:], pool, case.block_tables[0][2:], ok, case.num_pages, case.scale)
    assert rc == oracle.OK
    assert_close(got[2:].astype(np.float64), ref, TOL_FP32, "good sequence beside bad ones")
    # append: the bad sequences are left untouched, the good one appended
    dpool = to_dev_u8(pool)
    flags.zero_()
    bt_app = case.block_tables[0].copy()
    bt_app[1, 39 // 16] = case.num_pages   # the page the appended token of sequence 1 would go to
    binding.append_kv_rope_i8(None, to_dev_bf16(case.k_new[0]), to_dev_bf16(case.v_new[0]), dpool,
                              to_dev_i32(bt_app), to_dev_i32(lens), rope(), device_flags=flags)
    torch.cuda.synchronize()
    assert int(flags.item()) == binding.PA_DEVERR_CONTEXT_LEN | binding.PA_DEVERR_PAGE_ID
    got_pool = dpool.cpu().numpy()
    ref_pool = pool.copy()
    sel = [2]
    assert oracle.append_kv_rope_i8(None, case.k_new[0][sel], case.v_new[0][sel], ref_pool,
                                    case.block_tables[0][sel], case.context_lens[sel], case.num_pages,
                                    case.theta) == oracle.OK
    assert np.array_equal(got_pool, ref_pool)


def _full_size_i8(spec, layers, what):
    """The benchmark's INT8 step on whole layers of a full-size workload, every sequence checked
    against the oracle on bf16 pages copied to the host before any of our kernels ran."""
    k_pool = guarded_pool(spec, "k")
    v_pool = guarded_pool(spec, "v")
    seqs = np.arange(spec.num_seqs)
    host = []
    for layer in layers:
        bt = spec.block_tables[layer][seqs]
        used = np.unique(bt[bt >= 0])
        idx = torch.from_numpy(used).to(dev())
        kp = to_host_bits(k_pool.index_select(0, idx)).copy()   # bf16 pages, before any of our kernels
        vp = to_host_bits(v_pool.index_select(0, idx)).copy()
        remap = np.full(spec.num_pages, -1, np.int64)
        remap[used] = np.arange(len(used))
        bt_small = np.where(bt >= 0, remap[np.maximum(bt, 0)], -1).astype(np.int32)
        host.append((layer, used, idx, kp, vp, bt_small))
    pool = binding.i8_pool(spec.num_pages, dev())
    binding.quantize_pages_i8(pool, k_pool, v_pool)
    del k_pool, v_pool
    torch.cuda.empty_cache()
    table = rope(2048 + 64)
    ws = guarded_workspace(spec.num_seqs, spec.max_blocks)
    for layer, used, idx, kp, vp, bt_small in host:
        print(f"i8 full-size {what} layer={layer}: all {spec.num_seqs} sequences", flush=True)
        ref_pool = oracle.quantize_pages_i8(kp, vp)
        assert np.array_equal(pool.index_select(0, idx).cpu().numpy(), ref_pool)
        q, kn, vn = spec.host_rows(layer)
        dq = to_dev_bf16(q)
        out = guarded_empty((spec.num_seqs, 32, 64), torch.bfloat16)
        flags = guarded_flags()
        binding.append_decode_gqa_i8(out, dq, to_dev_bf16(kn), to_dev_bf16(vn), pool,
                                     to_dev_i32(spec.block_tables[layer]), to_dev_i32(spec.context_lens),
                                     table, spec.scale, workspace=ws, device_flags=flags)
        torch.cuda.synchronize()
        assert int(flags.item()) == 0
        lens = spec.context_lens.copy()
        oq = q.copy()
        assert oracle.append_kv_rope_i8(oq, kn.copy(), vn.copy(), ref_pool, bt_small, lens, len(used),
                                        spec.theta) == oracle.OK
        ref, rc = oracle.decode_gqa_i8(oq, ref_pool, bt_small, lens, len(used), spec.scale)
        assert rc == oracle.OK
        assert_close(to_host_f64(out), ref, TOL_BF16, f"{what} layer {layer}")
        assert_rope_equal(to_host_bits(dq), oq, "rotated q")
        # the pool after the append (the new K/V codes and scales), bit for bit
        assert np.array_equal(pool.index_select(0, idx).cpu().numpy(), ref_pool)
    del pool
    torch.cuda.empty_cache()


def test_batch64_i8_full_size_two_layers():
    """64 x 2048 tokens: the launch reads its codes with the non-temporal hint (512 workgroups)."""
    _full_size_i8(W.batch64_spec(), [0, 9], "batch64 i8")


def test_batch256_i8_full_size_one_layer():
    """The ragged, fragmented 256-sequence workload with 1 % outlier rows (2048 workgroups)."""
    _full_size_i8(W.batch256_spec(), [11], "batch256 i8")
