"""Full-size GPU parity, in the launch configuration the benchmark times.

The batch-64 x 2048 x 16-layer workload and the ragged batch-256 workload
(lognormal lengths, fragmented pool, 1% outlier rows x20) are built at full
size on the device.  Whole layers (two of batch-64, one of batch-256) run
through pa_append_decode_gqa exactly as the benchmark calls it, and every
sequence is checked against the fp64 oracle (append + decode).  The pages the
layer uses are copied to the host before the launch, so the oracle never sees
anything the HIP path wrote.  The rotated q rows and every used page
(appended K/V slots included) are compared bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from _gpu_helpers import TOL_BF16, assert_close, assert_rope_equal, dev, to_host_bits, to_host_f64
from _gpu_helpers import guarded_empty, guarded_flags, guarded_workspace, rope, guarded_pool, to_dev_i32, to_dev_bf16
from paged_kv_gqa_append_amd import binding
from paged_kv_gqa_append_amd import workloads as W

pytestmark = pytest.mark.gpu


def up(bits):
    return to_dev_bf16(bits)


def compact(spec, layer, seqs, k_pool, v_pool):
    """Host copy of the pages the sampled sequences use, with their tables remapped."""
    bt = spec.block_tables[layer][seqs]
    used = np.unique(bt[bt >= 0])
    remap = np.full(spec.num_pages, -1, np.int64)
    remap[used] = np.arange(len(used))
    idx = torch.from_numpy(used).to(dev())
    kp = to_host_bits(k_pool.index_select(0, idx)).copy()
    vp = to_host_bits(v_pool.index_select(0, idx)).copy()
    bt2 = np.where(bt >= 0, remap[np.maximum(bt, 0)], -1).astype(np.int32)
    return kp, vp, bt2, used


def run_case(spec, layers):
    """Every sequence of each listed layer, as the benchmark launches it."""
    k_pool = guarded_pool(spec, "k")
    v_pool = guarded_pool(spec, "v")
    seqs = np.arange(spec.num_seqs)
    table = rope(2048 + 64)
    ws = guarded_workspace(spec.num_seqs, spec.max_blocks)
    errs = []
    for layer in layers:
        print(f"full-size case={spec.name} layer={layer}: all {spec.num_seqs} sequences", flush=True)
        q, kn, vn = spec.host_rows(layer)
        kp, vp, bt_small, used = compact(spec, layer, seqs, k_pool, v_pool)  # before the launch
        dq = up(q)
        out = guarded_empty((spec.num_seqs, 32, 64), torch.bfloat16)
        flags = guarded_flags()
        binding.append_decode_gqa(out, dq, up(kn), up(vn), k_pool, v_pool,
                                  to_dev_i32(spec.block_tables[layer]),
                                  to_dev_i32(spec.context_lens), table, spec.scale,
                                  workspace=ws, device_flags=flags)
        torch.cuda.synchronize()
        assert int(flags.item()) == 0
        lens = spec.context_lens.copy()
        oq = q.copy()
        assert oracle.append_kv_rope(oq, kn.copy(), vn.copy(), kp, vp, bt_small, lens, len(used),
                                     spec.theta) == oracle.OK
        ref, rc = oracle.decode_gqa(oq, kp, vp, bt_small, lens, len(used), spec.scale)
        assert rc == oracle.OK
        errs.append(assert_close(to_host_f64(out), ref, TOL_BF16, f"{spec.name} layer {layer}"))
        # the rotated q rows and every page the layer uses (appended K/V slots included), bit for bit
        assert_rope_equal(to_host_bits(dq), oq, "rotated q")
        idx = torch.from_numpy(used).to(dev())
        assert_rope_equal(to_host_bits(k_pool.index_select(0, idx)), kp, "K pages")
        assert np.array_equal(to_host_bits(v_pool.index_select(0, idx)), vp)
    del k_pool, v_pool
    torch.cuda.empty_cache()
    return max(errs)


def test_batch64_full_size_two_layers():
    run_case(W.batch64_spec(), layers=[0, 15])


def test_batch256_ragged_full_size_one_layer():
    run_case(W.batch256_spec(), layers=[11])
