"""GPU parity of pa_append_decode_gqa (append + RoPE + decode in one launch).

Bar: bitwise equal to pa_append_kv_rope followed by pa_decode_gqa (pools, the
rotated q, the output in bf16 and fp32), and within the stated tolerance of the
oracle's append + decode.  Contexts above 2048 tokens exercise the
multi-partition path and its merge kernel.
"""
import numpy as np
import pytest
import torch

import oracle
from _gpu_helpers import TOL_BF16, TOL_FP32, DeviceCase, assert_close, dev, rope, to_dev_i32, to_host_bits, to_host_f64
from _gpu_helpers import guarded_empty, guarded_full, guarded_workspace
from paged_kv_gqa_append_amd import binding
from paged_kv_gqa_append_amd import workloads as W

pytestmark = pytest.mark.gpu

LONG = [2049, 3000, 4113, 17, 2048, 1]

CASES = {
    "tiny": lambda: W.tiny_decode(),
    "batch8": lambda: W.batch8_decode(),
    "edges": lambda: W.make_decode_case("edges", 61, [1, 2, 15, 16, 17, 255, 256, 257, 2047, 2048], dist="normal"),
    "long": lambda: W.make_decode_case("long", 62, LONG, dist="normal", max_blocks=260),
    "ragged_outliers": lambda: W.make_decode_case("ragged", 63, W.ragged_lengths(63, 20), dist="normal",
                                                  layout="fragmented", outlier_frac=0.01, max_blocks=128),
}


@pytest.fixture(scope="module")
def table():
    return rope(max_pos=4200)


def run_fused(case, table, out_dtype, alias=False):
    d = DeviceCase(case)
    ws = guarded_workspace(case.num_seqs, case.max_blocks)
    out = d.q if alias else guarded_empty((case.num_seqs, 32, 64), out_dtype)
    binding.append_decode_gqa(out, d.q, d.k_new, d.v_new, d.k_pool, d.v_pool, d.bt, d.lens, table, case.scale,
                              workspace=ws, device_flags=d.flags)
    torch.cuda.synchronize()
    return d, out


def run_separate(case, table, out_dtype):
    d = DeviceCase(case)
    ws = guarded_workspace(case.num_seqs, case.max_blocks)
    binding.append_kv_rope(d.q, d.k_new, d.v_new, d.k_pool, d.v_pool, d.bt, d.lens, table, device_flags=d.flags)
    out = guarded_empty((case.num_seqs, 32, 64), out_dtype)
    binding.decode_gqa(out, d.q, d.k_pool, d.v_pool, d.bt, d.lens, case.scale, workspace=ws, device_flags=d.flags)
    torch.cuda.synchronize()
    return d, out


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_fused_equals_separate_and_oracle(table, name, out_dtype):
    case = CASES[name]()
    if name == "tiny":
        case.context_lens[:] = 64
    print(f"fused case={name} B={case.num_seqs} out={out_dtype}", flush=True)
    fa, oa = run_fused(case, table, out_dtype)
    sb, ob = run_separate(case, table, out_dtype)
    assert int(fa.flags.item()) == 0 and int(sb.flags.item()) == 0
    assert np.array_equal(to_host_bits(fa.k_pool), to_host_bits(sb.k_pool)), "K pool differs"
    assert np.array_equal(to_host_bits(fa.v_pool), to_host_bits(sb.v_pool)), "V pool differs"
    assert np.array_equal(to_host_bits(fa.q), to_host_bits(sb.q)), "rotated q differs"
    got = to_host_f64(oa)
    assert np.array_equal(got, to_host_f64(ob)), "output differs from append-then-decode"
    kp, vp, q = case.k_pool.copy(), case.v_pool.copy(), case.q[0].copy()
    assert oracle.append_kv_rope(q, case.k_new[0], case.v_new[0], kp, vp, case.block_tables[0], case.context_lens,
                                 case.num_pages, case.theta) == oracle.OK
    ref, rc = oracle.decode_gqa(q, kp, vp, case.block_tables[0], case.context_lens, case.num_pages, case.scale)
    assert rc == oracle.OK
    assert_close(got, ref, TOL_BF16 if out_dtype == torch.bfloat16 else TOL_FP32, name)


@pytest.mark.parametrize("name", ["edges", "long"])
def test_fused_output_may_alias_q(table, name):
    case = CASES[name]()
    _, sep = run_fused(case, table, torch.bfloat16)
    d, out = run_fused(case, table, torch.bfloat16, alias=True)
    assert out.data_ptr() == d.q.data_ptr()
    assert np.array_equal(to_host_bits(out), to_host_bits(sep))


VERY_LONG = [32768, 20001, 1, 4097]


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_fused_very_long_contexts(out_dtype):
    """Contexts up to 32,768 tokens (16 partitions of 128 pages; 2,048-entry block-table rows, which
    validation reads in steps of the workgroup's 512 threads): fused equals append-then-decode bit
    for bit, and both are within tolerance of the oracle."""
    case = W.make_decode_case("very_long", 65, VERY_LONG, dist="normal", max_blocks=2048)
    table = rope(max_pos=32768 + 64)
    fa, oa = run_fused(case, table, out_dtype)
    sb, ob = run_separate(case, table, out_dtype)
    assert int(fa.flags.item()) == 0 and int(sb.flags.item()) == 0
    assert np.array_equal(to_host_bits(fa.k_pool), to_host_bits(sb.k_pool)), "K pool differs"
    assert np.array_equal(to_host_bits(fa.q), to_host_bits(sb.q)), "rotated q differs"
    got = to_host_f64(oa)
    assert np.array_equal(got, to_host_f64(ob)), "output differs from append-then-decode"
    kp, vp, q = case.k_pool.copy(), case.v_pool.copy(), case.q[0].copy()
    assert oracle.append_kv_rope(q, case.k_new[0], case.v_new[0], kp, vp, case.block_tables[0], case.context_lens,
                                 case.num_pages, case.theta) == oracle.OK
    ref, rc = oracle.decode_gqa(q, kp, vp, case.block_tables[0], case.context_lens, case.num_pages, case.scale)
    assert rc == oracle.OK
    assert_close(got, ref, TOL_BF16 if out_dtype == torch.bfloat16 else TOL_FP32, "very long")


def test_decode_long_contexts_against_oracle(table):
    case = CASES["long"]()
    d = DeviceCase(case)
    ws = guarded_workspace(case.num_seqs, case.max_blocks)
    assert ws is not None  # 260 blocks need more than one partition
    out = guarded_empty((case.num_seqs, 32, 64), torch.float32)
    binding.decode_gqa(out, d.q, d.k_pool, d.v_pool, d.bt, d.lens, case.scale, workspace=ws, device_flags=d.flags)
    torch.cuda.synchronize()
    ref, rc = oracle.decode_gqa(case.q[0], case.k_pool, case.v_pool, case.block_tables[0], case.context_lens,
                                case.num_pages, case.scale)
    assert rc == oracle.OK
    assert_close(to_host_f64(out), ref, TOL_FP32, "long")


def test_fused_device_errors(table):
    case = W.make_decode_case("err", 64, [40, 600, 17, 1000, 33], dist="normal", max_blocks=64)
    d = DeviceCase(case)
    lens = case.context_lens.copy()
    lens[0] = 0                 # bad length
    bt = case.block_tables[0].copy()
    bt[3, 40] = case.num_pages  # bad page in a used entry
    d.lens, d.bt = to_dev_i32(lens), to_dev_i32(bt)
    short = rope(max_pos=600)   # sequences 1 (pos 599 ok), 3 (pos 999) and ... beyond the table
    before_k = to_host_bits(d.k_pool)
    out = guarded_full((5, 32, 64), 7.0, torch.float32)
    binding.append_decode_gqa(out, d.q, d.k_new, d.v_new, d.k_pool, d.v_pool, d.bt, d.lens, short, case.scale,
                              device_flags=d.flags)
    torch.cuda.synchronize()
    assert int(d.flags.item()) == binding.PA_DEVERR_CONTEXT_LEN  # seq 3 fails on its position before its page
    got = to_host_f64(out)
    assert np.all(got[0] == 0) and np.all(got[3] == 0)
    # healthy sequences 1, 2, 4: compare with the oracle on those alone
    kp, vp, q = case.k_pool.copy(), case.v_pool.copy(), case.q[0].copy()
    oracle.append_kv_rope(q, case.k_new[0], case.v_new[0], kp, vp, case.block_tables[0], case.context_lens,
                          case.num_pages, case.theta)
    ref, _ = oracle.decode_gqa(q, kp, vp, case.block_tables[0], case.context_lens, case.num_pages, case.scale)
    for s in (1, 2, 4):
        assert_close(got[s], ref[s], TOL_FP32, f"seq {s}")
    # only the healthy sequences' slots were written
    gk = to_host_bits(d.k_pool)
    changed = {tuple(x) for x in np.argwhere(np.any(gk != before_k, axis=(1, 3)))}
    expect = {(case.block_tables[0, s, (case.context_lens[s] - 1) // 16], (case.context_lens[s] - 1) % 16)
              for s in (1, 2, 4)}
    assert changed == expect
    # a bad page id alone
    d2 = DeviceCase(case)
    d2.bt = to_dev_i32(bt)
    out2 = guarded_full((5, 32, 64), 7.0, torch.float32)
    binding.append_decode_gqa(out2, d2.q, d2.k_new, d2.v_new, d2.k_pool, d2.v_pool, d2.bt, d2.lens, table,
                              case.scale, device_flags=d2.flags)
    torch.cuda.synchronize()
    assert int(d2.flags.item()) == binding.PA_DEVERR_PAGE_ID
    assert np.all(to_host_f64(out2)[3] == 0)
