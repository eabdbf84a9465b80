"""Full-size GPU parity, in the launch configuration the benchmark times.

The batch-64 x 2048 x 16-layer workload and the ragged batch-256 workload
(lognormal lengths, fragmented pool, 1% outlier rows x20) are built at full
size on the device.  One layer runs through pa_append_decode_gqa exactly as
the benchmark calls it.  Sampled sequences are then checked against the fp64
oracle (append + decode) computed one by one.  The pages those sequences use
are copied to the host before the launch, so the oracle never sees anything
the HIP path wrote.  The appended K/V slots and the rotated q rows of the
sampled sequences are compared too.
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


def run_case(spec, layer, seqs):
    print(f"full-size case={spec.name} layer={layer} sampled={list(seqs)}", flush=True)
    k_pool = guarded_pool(spec, "k")
    v_pool = guarded_pool(spec, "v")
    q, kn, vn = spec.host_rows(layer)
    kp, vp, bt_small, used = compact(spec, layer, seqs, k_pool, v_pool)  # before the launch
    dq = up(q)
    out = guarded_empty((spec.num_seqs, 32, 64), torch.bfloat16)
    table = rope(2048 + 64)
    flags = guarded_flags()
    binding.append_decode_gqa(out, dq, up(kn), up(vn), k_pool, v_pool,
                              to_dev_i32(spec.block_tables[layer]),
                              to_dev_i32(spec.context_lens), table, spec.scale,
                              workspace=guarded_workspace(spec.num_seqs, spec.max_blocks),
                              device_flags=flags)
    torch.cuda.synchronize()
    assert int(flags.item()) == 0
    # oracle on the sampled sequences
    lens = spec.context_lens[seqs].copy()
    oq = q[seqs].copy()
    assert oracle.append_kv_rope(oq, kn[seqs].copy(), vn[seqs].copy(), kp, vp, bt_small, lens, len(used),
                                 spec.theta) == oracle.OK
    ref, rc = oracle.decode_gqa(oq, kp, vp, bt_small, lens, len(used), spec.scale)
    assert rc == oracle.OK
    got = to_host_f64(out)[seqs]
    err = assert_close(got, ref, TOL_BF16, spec.name)
    # rotated q and the appended K rows (1 ulp + fp32 bound), V rows exact
    assert_rope_equal(to_host_bits(dq)[seqs], oq, "rotated q")
    gk = to_host_bits(k_pool.index_select(0, torch.from_numpy(used).to(dev())))
    gv = to_host_bits(v_pool.index_select(0, torch.from_numpy(used).to(dev())))
    for i, L in enumerate(lens):
        pg, sl = bt_small[i, (L - 1) // 16], (L - 1) % 16
        assert_rope_equal(gk[pg, :, sl], kp[pg, :, sl], "appended K")
        assert np.array_equal(gv[pg, :, sl], vp[pg, :, sl])
    del k_pool, v_pool
    torch.cuda.empty_cache()
    return err


def test_batch64_full_size_sampled():
    spec = W.batch64_spec()
    run_case(spec, layer=5, seqs=np.array([0, 1, 17, 42, 63]))


def test_batch256_ragged_full_size_sampled():
    spec = W.batch256_spec()
    lens = spec.context_lens
    pick = sorted({int(np.argmin(lens)), int(np.argmax(lens)), int(np.argsort(lens)[len(lens) // 2]), 7, 200})
    run_case(spec, layer=11, seqs=np.array(pick))
