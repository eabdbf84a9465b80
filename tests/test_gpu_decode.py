"""GPU parity of pa_decode_gqa (and append + decode) against the fp64 oracle.

Bar (elementwise): bf16 out |gpu - ref| <= 1e-2 + 1e-2 |ref|, fp32 out
<= 2e-3 + 2e-3 |ref|.  Bitwise properties: one-token sequences return their V,
results do not depend on the batch, on page placement, or on the run, and the
output may overwrite q.  Every pool slot no sequence uses holds NaN.
"""
import numpy as np
import pytest
import torch

import oracle
from _gpu_helpers import (TOL_BF16, TOL_FP32, DeviceCase, assert_close, dev, rope, to_dev_bf16, to_dev_i32,
                          to_host_bits, to_host_f64)
from _gpu_helpers import guarded_empty, guarded_full, guarded_clone, guarded_workspace
from paged_kv_gqa_append_amd import binding
from paged_kv_gqa_append_amd import workloads as W

pytestmark = pytest.mark.gpu

EDGE = [1, 2, 15, 16, 17, 31, 33, 255, 256, 257, 511, 512, 513, 1023, 1024, 1025, 2047, 2048]


def gpu_decode(d: DeviceCase, out_dtype=torch.bfloat16, q=None, out=None):
    case = d.case
    q = d.q if q is None else q
    if out is None:
        out = guarded_empty((case.num_seqs, 32, 64), out_dtype)
    ws = guarded_workspace(case.num_seqs, case.max_blocks)
    binding.decode_gqa(out, q, d.k_pool, d.v_pool, d.bt, d.lens, case.scale, workspace=ws, device_flags=d.flags)
    torch.cuda.synchronize()
    return out


def oracle_decode(case, q_bits=None, layer=0):
    out, rc = oracle.decode_gqa(case.q[layer] if q_bits is None else q_bits, case.k_pool, case.v_pool,
                                case.block_tables[layer], case.context_lens, case.num_pages, case.scale)
    assert rc == oracle.OK
    return out


CASES = {
    "tiny": lambda: W.tiny_decode(),
    "batch8": lambda: W.batch8_decode(),
    "edges": lambda: W.make_decode_case("edges", 51, EDGE, dist="normal", max_blocks=130),
    "ragged_outliers": lambda: W.make_decode_case("ragged", 52, W.ragged_lengths(52, 24), dist="normal",
                                                  layout="fragmented", outlier_frac=0.01, max_blocks=128),
}


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_decode_parity(name, out_dtype):
    case = CASES[name]()
    print(f"decode parity case={name} B={case.num_seqs} out={out_dtype}", flush=True)
    d = DeviceCase(case)
    got = to_host_f64(gpu_decode(d, out_dtype))
    ref = oracle_decode(case)
    assert_close(got, ref, TOL_BF16 if out_dtype == torch.bfloat16 else TOL_FP32, name)
    assert int(d.flags.item()) == 0


@pytest.mark.parametrize("name", ["tiny", "batch8", "edges"])
def test_append_then_decode(name):
    case = CASES[name]()
    if name == "tiny":  # 63 cached tokens + the appended one at position 63
        case.context_lens[:] = 64
    table = rope()
    d = DeviceCase(case)
    binding.append_kv_rope(d.q, d.k_new, d.v_new, d.k_pool, d.v_pool, d.bt, d.lens, table, device_flags=d.flags)
    got = to_host_f64(gpu_decode(d, torch.float32))
    kp, vp, q = case.k_pool.copy(), case.v_pool.copy(), case.q[0].copy()
    assert oracle.append_kv_rope(q, case.k_new[0], case.v_new[0], kp, vp, case.block_tables[0], case.context_lens,
                                 case.num_pages, case.theta) == oracle.OK
    ref, rc = oracle.decode_gqa(q, kp, vp, case.block_tables[0], case.context_lens, case.num_pages, case.scale)
    assert rc == oracle.OK
    assert_close(got, ref, TOL_FP32, name)


def test_single_token_returns_v_bitwise():
    case = W.make_decode_case("one", 53, [1] * 5, dist="normal")
    d = DeviceCase(case)
    got = to_host_bits(gpu_decode(d, torch.bfloat16))
    for s in range(5):
        v = case.v_pool[case.block_tables[0, s, 0], :, 0, :]
        assert np.array_equal(got[s], np.repeat(v, 4, axis=0))


def test_identical_rows_and_ones_column():
    case = W.make_decode_case("same", 54, [700, 33, 1], dist="normal", max_blocks=64)
    row = W.f32_to_bf16_bits(np.random.default_rng(3).standard_normal((8, 64)).astype(np.float32))
    row[:, 7] = 0x3F80  # 1.0
    for s, L in enumerate(case.context_lens):
        for t in range(L):
            case.v_pool[case.block_tables[0, s, t // 16], :, t % 16, :] = row
    d = DeviceCase(case)
    got = to_host_f64(gpu_decode(d, torch.float32))
    ref = np.repeat(W.bf16_bits_to_f32(row).astype(np.float64), 4, axis=0)
    for s in range(3):
        assert_close(got[s], ref, (1e-6, 1e-6), "identical rows")
        assert np.all(np.abs(got[s, :, 7] - 1.0) < 1e-6)


def test_output_may_alias_q():
    case = CASES["edges"]()
    d = DeviceCase(case)
    sep = to_host_bits(gpu_decode(d, torch.bfloat16))
    q_alias = guarded_clone(d.q)
    gpu_decode(d, torch.bfloat16, q=q_alias, out=q_alias)
    assert np.array_equal(to_host_bits(q_alias), sep)


def test_batch_invariance_and_determinism():
    case = CASES["edges"]()
    d = DeviceCase(case)
    full = to_host_bits(gpu_decode(d, torch.bfloat16))
    again = to_host_bits(gpu_decode(d, torch.bfloat16))
    assert np.array_equal(full, again), "run-to-run difference"
    # each sequence alone, and the batch reversed
    for s in [0, 5, 9, 17]:
        sub = W.PagedCase(name="one", num_layers=1, num_seqs=1, max_blocks=case.max_blocks,
                          num_pages=case.num_pages, context_lens=case.context_lens[s:s + 1].copy(),
                          block_tables=case.block_tables[:, s:s + 1].copy(), q=case.q[:, s:s + 1].copy(),
                          k_new=case.k_new[:, s:s + 1].copy(), v_new=case.v_new[:, s:s + 1].copy(),
                          k_pool=case.k_pool, v_pool=case.v_pool)
        alone = to_host_bits(gpu_decode(DeviceCase(sub), torch.bfloat16))
        assert np.array_equal(alone[0], full[s]), f"sequence {s} differs alone vs in batch"
    rev = W.PagedCase(name="rev", num_layers=1, num_seqs=case.num_seqs, max_blocks=case.max_blocks,
                      num_pages=case.num_pages, context_lens=case.context_lens[::-1].copy(),
                      block_tables=case.block_tables[:, ::-1].copy(), q=case.q[:, ::-1].copy(),
                      k_new=case.k_new[:, ::-1].copy(), v_new=case.v_new[:, ::-1].copy(),
                      k_pool=case.k_pool, v_pool=case.v_pool)
    assert np.array_equal(to_host_bits(gpu_decode(DeviceCase(rev), torch.bfloat16))[::-1], full)


def test_page_permutation_bitwise():
    case = CASES["edges"]()
    base = to_host_f64(gpu_decode(DeviceCase(case), torch.float32))
    perm = np.random.default_rng(7).permutation(case.num_pages)
    kp = np.empty_like(case.k_pool)
    vp = np.empty_like(case.v_pool)
    kp[perm] = case.k_pool
    vp[perm] = case.v_pool
    bt = np.where(case.block_tables >= 0, perm[np.maximum(case.block_tables, 0)], -1).astype(np.int32)
    moved = W.PagedCase(name="perm", num_layers=1, num_seqs=case.num_seqs, max_blocks=case.max_blocks,
                        num_pages=case.num_pages, context_lens=case.context_lens, block_tables=bt, q=case.q,
                        k_new=case.k_new, v_new=case.v_new, k_pool=kp, v_pool=vp)
    got = to_host_f64(gpu_decode(DeviceCase(moved), torch.float32))
    assert np.array_equal(got, base)


def test_device_errors_zero_fill_and_flag():
    case = W.make_decode_case("err", 55, [40, 600, 17, 1000], dist="normal", max_blocks=64)
    ref = oracle_decode(case)
    d = DeviceCase(case)
    lens = case.context_lens.copy()
    lens[0] = 0                 # bad length
    lens[2] = 64 * 16 + 1       # beyond the table
    bt = case.block_tables[0].copy()
    bt[3, 40] = -1              # a used entry of a multi-partition sequence
    d.lens, d.bt = to_dev_i32(lens), to_dev_i32(bt)
    out = guarded_full((4, 32, 64), 7.0, torch.float32)
    gpu_decode(d, out=out)
    got = to_host_f64(out)
    assert int(d.flags.item()) == binding.PA_DEVERR_CONTEXT_LEN | binding.PA_DEVERR_PAGE_ID
    assert np.all(got[0] == 0) and np.all(got[2] == 0) and np.all(got[3] == 0)
    assert_close(got[1], ref[1], TOL_FP32, "healthy sequence next to bad ones")


def test_device_error_read_back():
    """pa_get_device_error returns the bits a kernel flagged (after draining the stream), resets
    the word when asked, and reads 0 after a clean call."""
    case = W.make_decode_case("err_rb", 56, [40, 600, 17], dist="normal", max_blocks=64)
    d = DeviceCase(case)
    out = guarded_empty((3, 32, 64), torch.bfloat16)
    gpu_decode(d, out=out)  # clean
    assert binding.get_device_error(d.flags) == 0
    bt = case.block_tables[0].copy()
    bt[1, 7] = case.num_pages + 3  # a used page id outside the pool
    d.bt = to_dev_i32(bt)
    gpu_decode(d, out=out)
    assert binding.get_device_error(d.flags) == binding.PA_DEVERR_PAGE_ID
    assert binding.get_device_error(d.flags, clear=True) == binding.PA_DEVERR_PAGE_ID
    assert binding.get_device_error(d.flags) == 0
    lens = case.context_lens.copy()
    lens[2] = 0
    d.lens, d.bt = to_dev_i32(lens), to_dev_i32(case.block_tables[0])
    gpu_decode(d, out=out)
    assert binding.get_device_error(d.flags, clear=True) == binding.PA_DEVERR_CONTEXT_LEN
    assert int(d.flags.item()) == 0
