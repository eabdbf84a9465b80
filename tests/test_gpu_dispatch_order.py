"""A dispatch order changes which workgroups start first and nothing else: the
same batch launched in slot order, longest first and in a seeded random order
gives the same bits (decode, and append + decode: out, the rotated q and the
pools), for bf16 and INT8 pages.  The batch is ragged and two of its sequences
run past one 2048-token partition, so the order's items carry partition
numbers too; the ordered outputs also meet the oracle's tolerance."""
import numpy as np
import pytest
import torch

import oracle
from _gpu_helpers import TOL_BF16, assert_close, dev, rope, to_dev_bf16, to_dev_i32, to_host_bits
from _gpu_helpers import guarded_empty, guarded_workspace, to_dev_u8
from paged_kv_gqa_append_amd import binding
from paged_kv_gqa_append_amd import workloads as W

pytestmark = pytest.mark.gpu


def make_case():
    rng = np.random.default_rng(91)
    lens = np.clip(np.rint(np.exp(rng.normal(6.0, 1.0, size=40))), 1, 2048).astype(np.int32)
    lens[:2] = [3000, 4095]  # two sequences past one partition (max_blocks 256: two partitions each)
    return W.make_decode_case("order40", 92, lens, dist="normal", max_blocks=256)


def run(case, kv, fused, order, host_i8, table):
    if kv == "int8":
        pools = [to_dev_u8(host_i8)]
    else:
        pools = [to_dev_bf16(case.k_pool), to_dev_bf16(case.v_pool)]
    q = to_dev_bf16(case.q[0])
    bt, lens = to_dev_i32(case.block_tables[0]), to_dev_i32(case.context_lens)
    kn, vn = to_dev_bf16(case.k_new[0]), to_dev_bf16(case.v_new[0])
    out = guarded_empty((case.num_seqs, 32, 64), torch.bfloat16)
    ws = guarded_workspace(case.num_seqs, case.max_blocks)
    if kv == "int8":
        if fused:
            binding.append_decode_gqa_i8(out, q, kn, vn, pools[0], bt, lens, table, case.scale, workspace=ws,
                                         dispatch_order=order)
        else:
            binding.decode_gqa_i8(out, q, pools[0], bt, lens, case.scale, workspace=ws, dispatch_order=order)
    else:
        if fused:
            binding.append_decode_gqa(out, q, kn, vn, pools[0], pools[1], bt, lens, table, case.scale, workspace=ws,
                                      dispatch_order=order)
        else:
            binding.decode_gqa(out, q, pools[0], pools[1], bt, lens, case.scale, workspace=ws, dispatch_order=order)
    torch.cuda.synchronize()
    return to_host_bits(out), to_host_bits(q), [p.view(torch.uint8).cpu().numpy() for p in pools]


@pytest.mark.parametrize("kv", ["bf16", "int8"])
@pytest.mark.parametrize("fused", [False, True])
def test_ordered_launches_agree_bitwise(kv, fused):
    print(f"dispatch order: kv={kv} fused={fused}", flush=True)
    case = make_case()
    host_i8 = oracle.quantize_pages_i8(case.k_pool, case.v_pool) if kv == "int8" else None
    table = rope()
    base = run(case, kv, fused, None, host_i8, table)
    orders = {"longest first": np.argsort(-case.context_lens, kind="stable"),
              "random": np.random.default_rng(93).permutation(case.num_seqs)}
    for name, order in orders.items():
        got = run(case, kv, fused, order, host_i8, table)
        assert np.array_equal(base[0], got[0]), f"{name}: out differs"
        if fused:
            assert np.array_equal(base[1], got[1]), f"{name}: rotated q differs"
            for a, b in zip(base[2], got[2]):
                assert np.array_equal(a, b), f"{name}: pool differs after the append"
    if not fused:  # the decode-only calls attend with the q as given
        if kv == "int8":
            ref, rc = oracle.decode_gqa_i8(case.q[0], host_i8, case.block_tables[0], case.context_lens,
                                           case.num_pages, case.scale)
        else:
            ref, rc = oracle.decode_gqa(case.q[0], case.k_pool, case.v_pool, case.block_tables[0],
                                        case.context_lens, case.num_pages, case.scale)
        assert rc == oracle.OK
        assert_close(W.bf16_bits_to_f32(got[0]).astype(np.float64), ref, TOL_BF16, f"{kv} ordered")
