"""GPU parity of pa_append_kv_rope against the oracle.

Bar: every byte of both pools and of the rotated q bit-identical to the
oracle's result (the device rotates with the oracle's fp64 operations), and so
which slots are written (the indexing).
"""
import numpy as np
import pytest
import torch

import oracle
from _gpu_helpers import DeviceCase, assert_rope_equal, dev, rope, to_dev_i32, to_host_bits
from _gpu_helpers import guarded_flags
from paged_kv_gqa_append_amd import binding
from paged_kv_gqa_append_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def table():
    return rope()


def run_both(case, table, with_q=True):
    d = DeviceCase(case)
    binding.append_kv_rope(d.q if with_q else None, d.k_new, d.v_new, d.k_pool, d.v_pool, d.bt, d.lens, table,
                           device_flags=d.flags)
    torch.cuda.synchronize()
    kp, vp, q = case.k_pool.copy(), case.v_pool.copy(), case.q[0].copy()
    rc = oracle.append_kv_rope(q if with_q else None, case.k_new[0], case.v_new[0], kp, vp, case.block_tables[0],
                               case.context_lens, case.num_pages, case.theta)
    assert rc == oracle.OK
    return d, kp, vp, q


def check(case, d, kp, vp, q, with_q=True):
    gk, gv, gq = to_host_bits(d.k_pool), to_host_bits(d.v_pool), to_host_bits(d.q)
    assert np.array_equal(gv, vp), "V pool differs from the oracle"
    diff = gk != kp
    # where the two differ from the pool they started from: the appended slots only
    appended = np.zeros(kp.shape[0:1] + (16,), bool)
    for s, L in enumerate(case.context_lens):
        appended[case.block_tables[0, s, (L - 1) // 16], (L - 1) % 16] = True
    assert not np.any(diff.transpose(0, 2, 1, 3)[~appended]), "bytes outside the appended slots changed"
    assert_rope_equal(gk, kp, "K pool")
    # the appended slots really changed (they held NaN poison or other data)
    assert np.array_equal(np.any(gk != case.k_pool, axis=(1, 3)), appended)
    if with_q:
        assert_rope_equal(gq, q, "rotated q")
    else:
        assert np.array_equal(gq, case.q[0])
    assert int(d.flags.item()) == 0


@pytest.mark.parametrize("name", ["tiny", "batch8", "edges", "long"])
def test_append_parity(table, name):
    if name == "tiny":
        case = W.tiny_decode()
    elif name == "batch8":
        case = W.batch8_decode()
    elif name == "edges":
        case = W.make_decode_case("edges", 41, [1, 2, 15, 16, 17, 32, 33, 255, 256, 257], dist="normal")
    else:
        case = W.make_decode_case("long", 42, [2047, 2048, 1024, 1025, 511], dist="normal")
    print(f"append parity case={name} B={case.num_seqs}", flush=True)
    d, kp, vp, q = run_both(case, table)
    check(case, d, kp, vp, q)


def test_append_without_q(table):
    case = W.make_decode_case("noq", 43, [5, 80, 16], dist="normal")
    d, kp, vp, q = run_both(case, table, with_q=False)
    check(case, d, kp, vp, q, with_q=False)


def test_append_outlier_magnitudes(table):
    case = W.make_decode_case("big", 44, [9, 300], dist="normal")
    case.k_new[:] = W.f32_to_bf16_bits(W.bf16_bits_to_f32(case.k_new) * 20.0)
    d, kp, vp, q = run_both(case, table)
    check(case, d, kp, vp, q)


def test_append_device_errors_leave_pool_untouched(table):
    case = W.make_decode_case("err", 45, [10, 20, 30], dist="normal")
    d = DeviceCase(case)
    lens = case.context_lens.copy()
    lens[0] = 0                       # bad length
    bt = case.block_tables[0].copy()
    bt[1, (20 - 1) // 16] = case.num_pages + 3  # bad page id for seq 1
    d.lens = to_dev_i32(lens)
    d.bt = to_dev_i32(bt)
    before_k, before_v = to_host_bits(d.k_pool), to_host_bits(d.v_pool)
    binding.append_kv_rope(d.q, d.k_new, d.v_new, d.k_pool, d.v_pool, d.bt, d.lens, table, device_flags=d.flags)
    torch.cuda.synchronize()
    assert int(d.flags.item()) == binding.PA_DEVERR_CONTEXT_LEN | binding.PA_DEVERR_PAGE_ID
    gk, gv = to_host_bits(d.k_pool), to_host_bits(d.v_pool)
    page2 = case.block_tables[0, 2, (30 - 1) // 16]
    changed = np.argwhere(np.any(gk != before_k, axis=(1, 3)))
    assert [tuple(x) for x in changed] == [(page2, (30 - 1) % 16)]
    assert np.array_equal(np.any(gv != before_v, axis=(1, 3)), np.any(gk != before_k, axis=(1, 3)))
    # q rows of the failed sequences untouched, seq 2 rotated
    gq = to_host_bits(d.q)
    assert np.array_equal(gq[0], case.q[0, 0]) and np.array_equal(gq[1], case.q[0, 1])
    # position beyond the rope table is a length error as well
    short = rope(max_pos=16)
    f2 = guarded_flags()
    binding.append_kv_rope(None, d.k_new, d.v_new, d.k_pool, d.v_pool, to_dev_i32(case.block_tables[0]),
                           to_dev_i32(case.context_lens), short, device_flags=f2)
    torch.cuda.synchronize()
    assert int(f2.item()) == binding.PA_DEVERR_CONTEXT_LEN
