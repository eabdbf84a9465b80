"""Child process of test_gpu_partition_sweep: the decode partition size is read
from PA_DECODE_PART_PAGES once per process, so each size runs in a process of
its own.  Checks decode and append + decode, bf16 and INT8 pages, against the
oracle on a case whose sequences span several partitions at that size; prints
one JSON line and exits 0 on success."""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

import numpy as np  # noqa: E402
import torch  # noqa: E402

import oracle  # noqa: E402
from _gpu_helpers import TOL_BF16, TOL_FP32, DeviceCase, assert_close, dev, rope, to_dev_bf16, to_dev_i32, to_host_f64  # noqa: E402,E501
from _gpu_helpers import guarded_empty, guarded_workspace, to_dev_u8, check_guards  # noqa: E402
from paged_kv_gqa_append_amd import binding  # noqa: E402
from paged_kv_gqa_append_amd import workloads as W  # noqa: E402


def main():
    part_tokens = binding.decode_partition_tokens()
    want = int(os.environ["PA_DECODE_PART_PAGES"]) * 16
    assert part_tokens == want, (part_tokens, want)
    lens = [1, 16, 17, 129, 500, 1023, 2048, 2049, 3000]
    case = W.make_decode_case("sweep", 81, lens, dist="normal", max_blocks=200)
    table = rope(max_pos=3300)
    ws = guarded_workspace(case.num_seqs, case.max_blocks)
    # bf16: decode alone (fp32 out) and append + decode (bf16 out)
    d = DeviceCase(case)
    out = guarded_empty((case.num_seqs, 32, 64), torch.float32)
    binding.decode_gqa(out, d.q, d.k_pool, d.v_pool, d.bt, d.lens, case.scale, workspace=ws, device_flags=d.flags)
    torch.cuda.synchronize()
    ref, rc = oracle.decode_gqa(case.q[0], case.k_pool, case.v_pool, case.block_tables[0], case.context_lens,
                                case.num_pages, case.scale)
    assert rc == oracle.OK and int(d.flags.item()) == 0
    assert_close(to_host_f64(out), ref, TOL_FP32, f"bf16 decode, partition {part_tokens}")
    d = DeviceCase(case)
    out = guarded_empty((case.num_seqs, 32, 64), torch.bfloat16)
    binding.append_decode_gqa(out, d.q, d.k_new, d.v_new, d.k_pool, d.v_pool, d.bt, d.lens, table, case.scale,
                              workspace=ws, device_flags=d.flags)
    torch.cuda.synchronize()
    kp, vp, q = case.k_pool.copy(), case.v_pool.copy(), case.q[0].copy()
    assert oracle.append_kv_rope(q, case.k_new[0], case.v_new[0], kp, vp, case.block_tables[0], case.context_lens,
                                 case.num_pages, case.theta) == oracle.OK
    ref, rc = oracle.decode_gqa(q, kp, vp, case.block_tables[0], case.context_lens, case.num_pages, case.scale)
    assert rc == oracle.OK and int(d.flags.item()) == 0
    assert_close(to_host_f64(out), ref, TOL_BF16, f"bf16 append + decode, partition {part_tokens}")
    # INT8: append + decode (fp32 out)
    pool_h = oracle.quantize_pages_i8(case.k_pool, case.v_pool)
    pool = to_dev_u8(pool_h)
    out = guarded_empty((case.num_seqs, 32, 64), torch.float32)
    binding.append_decode_gqa_i8(out, to_dev_bf16(case.q[0]), to_dev_bf16(case.k_new[0]), to_dev_bf16(case.v_new[0]),
                                 pool, to_dev_i32(case.block_tables[0]), to_dev_i32(case.context_lens), table,
                                 case.scale, workspace=ws)
    torch.cuda.synchronize()
    oq, opool = case.q[0].copy(), pool_h.copy()
    assert oracle.append_kv_rope_i8(oq, case.k_new[0], case.v_new[0], opool, case.block_tables[0],
                                    case.context_lens, case.num_pages, case.theta) == oracle.OK
    ref, rc = oracle.decode_gqa_i8(oq, opool, case.block_tables[0], case.context_lens, case.num_pages, case.scale)
    assert rc == oracle.OK
    assert_close(to_host_f64(out), ref, TOL_FP32, f"INT8 append + decode, partition {part_tokens}")
    check_guards()
    print(json.dumps({"partition_tokens": part_tokens, "ok": True}), flush=True)


if __name__ == "__main__":
    main()
