"""The decode kernels choose their page-load form by grid size (one workgroup
per sequence and KV head here).  bf16: from 128 workgroups, whole-row loads
with the non-temporal hint, whose registers are put in the lane's slot order
by selects; below, plain loads straight into slot order.  INT8: the hint on
the code loads from 128 workgroups, and wave priorities levelled only up to
1024.  None of this changes any arithmetic: a batch that takes one form and
the same sequences split into batches that take the other give the same bits
(decode, and append + decode: out, the rotated q and the pool), and the
larger batch matches the oracle."""
import numpy as np
import pytest
import torch

import oracle
from _gpu_helpers import TOL_BF16, assert_close, dev, rope, to_dev_bf16, to_dev_i32, to_host_bits
from _gpu_helpers import guarded_empty, guarded_workspace, to_dev_u8
from paged_kv_gqa_append_amd import binding
from paged_kv_gqa_append_amd import workloads as W

pytestmark = pytest.mark.gpu


def sub_case(case, lo, hi):
    return W.PagedCase(name=f"{case.name}[{lo}:{hi}]", num_layers=1, num_seqs=hi - lo, max_blocks=case.max_blocks,
                       num_pages=case.num_pages, context_lens=case.context_lens[lo:hi].copy(),
                       block_tables=case.block_tables[:, lo:hi].copy(), q=case.q[:, lo:hi].copy(),
                       k_new=case.k_new[:, lo:hi].copy(), v_new=case.v_new[:, lo:hi].copy(),
                       k_pool=case.k_pool, v_pool=case.v_pool, scale=case.scale, seed=case.seed)


def run(case, kv, fused, pools, table):
    """One call over all of case's sequences on the given device pools (modified in place when
    fused); returns (out bits, q bits)."""
    q = to_dev_bf16(case.q[0])
    bt, lens = to_dev_i32(case.block_tables[0]), to_dev_i32(case.context_lens)
    kn, vn = to_dev_bf16(case.k_new[0]), to_dev_bf16(case.v_new[0])
    out = guarded_empty((case.num_seqs, 32, 64), torch.bfloat16)
    ws = guarded_workspace(case.num_seqs, case.max_blocks)
    if kv == "int8":
        if fused:
            binding.append_decode_gqa_i8(out, q, kn, vn, pools[0], bt, lens, table, case.scale, workspace=ws)
        else:
            binding.decode_gqa_i8(out, q, pools[0], bt, lens, case.scale, workspace=ws)
    else:
        if fused:
            binding.append_decode_gqa(out, q, kn, vn, pools[0], pools[1], bt, lens, table, case.scale,
                                      workspace=ws)
        else:
            binding.decode_gqa(out, q, pools[0], pools[1], bt, lens, case.scale, workspace=ws)
    torch.cuda.synchronize()
    return to_host_bits(out), to_host_bits(q)


def device_pools(case, kv, host_i8):
    if kv == "int8":
        return [to_dev_u8(host_i8)]
    return [to_dev_bf16(case.k_pool), to_dev_bf16(case.v_pool)]


# (kv, number of sequences of the whole batch, split point): the whole batch and its parts fall on
# opposite sides of a hint threshold.
SPLITS = [("bf16", 16, 8),      # 128 workgroups (whole rows) vs 2 x 64 (slot order)
          ("bf16", 20, 15),     # 160 (whole rows) vs 120 + 40 (slot order)
          ("int8", 16, 8),      # 128 (hinted) vs 2 x 64 (plain)
          ("int8", 130, 65)]    # 1040 (hinted, no priority levelling) vs 2 x 520 (hinted, levelled)


@pytest.mark.parametrize("kv,n,cut", SPLITS)
@pytest.mark.parametrize("fused", [False, True])
def test_hinted_and_plain_launches_agree_bitwise(kv, n, cut, fused):
    print(f"load hint: kv={kv} seqs={n} split={cut} fused={fused}", flush=True)
    rng = np.random.default_rng(60 + n)
    lens = rng.integers(1, 300 if n > 64 else 2049, size=n).astype(np.int32)
    lens[:3] = [1, 16, 2048 if n <= 64 else 299]
    case = W.make_decode_case(f"hint{n}", 61 + n, lens, dist="normal", max_blocks=128)
    host_i8 = oracle.quantize_pages_i8(case.k_pool, case.v_pool) if kv == "int8" else None
    table = rope()
    whole_pools = device_pools(case, kv, host_i8)
    whole_out, whole_q = run(case, kv, fused, whole_pools, table)
    part_pools = device_pools(case, kv, host_i8)
    outs, qs = [], []
    for lo, hi in ((0, cut), (cut, n)):
        o, q = run(sub_case(case, lo, hi), kv, fused, part_pools, table)
        outs.append(o)
        qs.append(q)
    assert np.array_equal(whole_out, np.concatenate(outs)), "out differs between hinted and plain launches"
    if fused:
        assert np.array_equal(whole_q, np.concatenate(qs)), "rotated q differs"
        for a, b in zip(whole_pools, part_pools):  # bit patterns: unused slots hold NaN
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), "pool differs after the append"
    else:
        # against the oracle (the decode-only calls attend with the q as given)
        if kv == "int8":
            ref, rc = oracle.decode_gqa_i8(case.q[0], host_i8, case.block_tables[0], case.context_lens,
                                           case.num_pages, case.scale)
        else:
            ref, rc = oracle.decode_gqa(case.q[0], case.k_pool, case.v_pool, case.block_tables[0],
                                        case.context_lens, case.num_pages, case.scale)
        assert rc == oracle.OK
        got = W.bf16_bits_to_f32(whole_out).astype(np.float64)
        assert_close(got, ref, TOL_BF16, f"{kv} {n}")
