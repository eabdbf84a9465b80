"""GPU parity for softmax scales other than 1/sqrt(64): negative (the scores' order reverses; the
prefill kernel negates q for its products), zero (every live key weighs the same: the plain
average of V) and large (4.0: sharply peaked weights, so the running reference moves often).
Decode over bf16 and INT8 pages, fused append + decode, and chunked prefill into bf16 and INT8
pages, each against the oracle evaluated with the same scale, within the fp32 tolerance."""
import numpy as np
import pytest
import torch

import oracle
from _gpu_helpers import (TOL_FP32, DeviceCase, assert_close, guarded_empty, guarded_flags, guarded_workspace, rope,
                          to_dev_bf16, to_dev_i32, to_dev_u8, to_host_f64)
from paged_kv_gqa_append_amd import binding
from paged_kv_gqa_append_amd import workloads as W

pytestmark = pytest.mark.gpu

SCALES = [-0.125, 0.0, 4.0]
LENS = [1, 17, 300, 2049]


def decode_case():
    return W.make_decode_case("scale", 90, LENS, dist="normal", max_blocks=130)


@pytest.mark.parametrize("scale", SCALES)
def test_decode_scales(scale):
    case = decode_case()
    d = DeviceCase(case)
    out = guarded_empty((case.num_seqs, 32, 64), torch.float32)
    binding.decode_gqa(out, d.q, d.k_pool, d.v_pool, d.bt, d.lens, scale,
                       workspace=guarded_workspace(case.num_seqs, case.max_blocks), device_flags=d.flags)
    torch.cuda.synchronize()
    assert int(d.flags.item()) == 0
    ref, rc = oracle.decode_gqa(case.q[0], case.k_pool, case.v_pool, case.block_tables[0], case.context_lens,
                                case.num_pages, scale)
    assert rc == oracle.OK
    assert_close(to_host_f64(out), ref, TOL_FP32, f"decode, scale {scale}")


@pytest.mark.parametrize("scale", SCALES)
def test_fused_scales(scale):
    case = decode_case()
    d = DeviceCase(case)
    out = guarded_empty((case.num_seqs, 32, 64), torch.float32)
    binding.append_decode_gqa(out, d.q, d.k_new, d.v_new, d.k_pool, d.v_pool, d.bt, d.lens, rope(max_pos=4200),
                              scale, workspace=guarded_workspace(case.num_seqs, case.max_blocks),
                              device_flags=d.flags)
    torch.cuda.synchronize()
    assert int(d.flags.item()) == 0
    kp, vp, q = case.k_pool.copy(), case.v_pool.copy(), case.q[0].copy()
    assert oracle.append_kv_rope(q, case.k_new[0], case.v_new[0], kp, vp, case.block_tables[0], case.context_lens,
                                 case.num_pages, case.theta) == oracle.OK
    ref, rc = oracle.decode_gqa(q, kp, vp, case.block_tables[0], case.context_lens, case.num_pages, scale)
    assert rc == oracle.OK
    assert_close(to_host_f64(out), ref, TOL_FP32, f"fused, scale {scale}")


@pytest.mark.parametrize("scale", SCALES)
def test_decode_i8_scales(scale):
    case = decode_case()
    pool = oracle.quantize_pages_i8(case.k_pool, case.v_pool)
    out = guarded_empty((case.num_seqs, 32, 64), torch.float32)
    flags = guarded_flags()
    binding.decode_gqa_i8(out, to_dev_bf16(case.q[0]), to_dev_u8(pool),
                          to_dev_i32(case.block_tables[0]), to_dev_i32(case.context_lens), scale,
                          workspace=guarded_workspace(case.num_seqs, case.max_blocks), device_flags=flags)
    torch.cuda.synchronize()
    assert int(flags.item()) == 0
    ref, rc = oracle.decode_gqa_i8(case.q[0], pool, case.block_tables[0], case.context_lens, case.num_pages, scale)
    assert rc == oracle.OK
    assert_close(to_host_f64(out), ref, TOL_FP32, f"INT8 decode, scale {scale}")


@pytest.mark.parametrize("scale", SCALES)
def test_prefill_scales(scale):
    c = W.make_prefill_case("scale", 91, [5, 40, 300], 37, poison=True)
    q = to_dev_bf16(c.q)
    kp, vp = to_dev_bf16(c.k_pool), to_dev_bf16(c.v_pool)
    flags = guarded_flags()
    out = guarded_empty(q.shape, torch.float32)
    binding.prefill_chunk(out, q, to_dev_bf16(c.k_chunk), to_dev_bf16(c.v_chunk), kp, vp, to_dev_i32(c.block_tables),
                          to_dev_i32(c.prefix_lens), rope(max_pos=4200), scale, device_flags=flags)
    torch.cuda.synchronize()
    assert int(flags.item()) == 0
    qh, kph, vph = c.q.copy(), c.k_pool.copy(), c.v_pool.copy()
    ref, rc = oracle.prefill_chunk(qh, c.k_chunk, c.v_chunk, kph, vph, c.block_tables, c.prefix_lens, c.num_pages,
                                   c.theta, scale)
    assert rc == oracle.OK
    assert_close(to_host_f64(out), ref, TOL_FP32, f"prefill, scale {scale}")


@pytest.mark.parametrize("scale", SCALES)
def test_prefill_i8_scales(scale):
    """Chunked prefill into INT8 pages: the scale reaches the scores through the per-key K scale
    products, so a negative scale flips every score's sign there."""
    c = W.make_prefill_case("scale8", 92, [5, 40, 300], 37, poison=True)
    pool = oracle.quantize_pages_i8(c.k_pool, c.v_pool)
    q = to_dev_bf16(c.q)
    flags = guarded_flags()
    out = guarded_empty(q.shape, torch.float32)
    binding.prefill_chunk_i8(out, q, to_dev_bf16(c.k_chunk), to_dev_bf16(c.v_chunk), to_dev_u8(pool),
                             to_dev_i32(c.block_tables), to_dev_i32(c.prefix_lens), rope(max_pos=4200), scale,
                             device_flags=flags)
    torch.cuda.synchronize()
    assert int(flags.item()) == 0
    qh, ph = c.q.copy(), pool.copy()
    ref, rc = oracle.prefill_chunk_i8(qh, c.k_chunk, c.v_chunk, ph, c.block_tables, c.prefix_lens, c.num_pages,
                                      c.theta, scale)
    assert rc == oracle.OK
    assert_close(to_host_f64(out), ref, TOL_FP32, f"INT8 prefill, scale {scale}")
