"""GPU parity of a multi-step decode loop driven by the host page manager.

Requests are queued in the pa_kvm manager; admitted ones get their prompt
written by pa_prefill_chunk, then decode one token per step with
pa_append_decode_gqa until their budget (prompt + max_new - 1 tokens) is full;
finished slots are released and queued requests admitted into the recycled
pages (samir-vllm, section "Gestion de la KV cache et strategies de batching":
pages are filled at prefill, each decoded token is appended at its absolute
RoPE position, requests are admitted as budgets free up).  Sequences cross
page boundaries and reuse fragmented pages.  Every step's outputs are
compared with the fp64 oracle running the same calls on its own host copy of
the pool, and at the end the pools themselves: V bit-exact, K within the
rotated-row bound.
"""
import numpy as np
import pytest
import torch

import oracle
from _gpu_helpers import (TOL_BF16, assert_close, assert_rope_equal, dev, rope, to_dev_bf16, to_dev_i32,
                          to_host_bits, to_host_f64)
from _gpu_helpers import guarded_empty, guarded_flags, guarded_workspace
from paged_kv_gqa_append_amd import binding
from paged_kv_gqa_append_amd import workloads as W

pytestmark = pytest.mark.gpu

P, LAYERS, SLOTS, MB = 24, 2, 4, 8  # 24 pages: admissions wait for budgets
SCALE = 0.125
REQUESTS = [(20, 30), (33, 14), (1, 40), (15, 20), (50, 10), (5, 60), (16, 17)]


def bf16(rng, shape):
    return W.f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32))


@pytest.mark.parametrize("batching", [binding.PA_BATCH_CONTINUOUS, binding.PA_BATCH_STATIC])
def test_manager_driven_decode_loop(batching):
    rng = np.random.default_rng(90 + batching)
    table = rope(max_pos=MB * 16 + 8)
    m = binding.KVManager(P, LAYERS, SLOTS, MB, batching=batching)
    for prompt, new in REQUESTS:
        m.submit(prompt, new)
    # both sides start from the same random pool contents (unused slots hold noise)
    kp_host = bf16(rng, (P, 8, 16, 64))
    vp_host = bf16(rng, (P, 8, 16, 64))
    kp, vp = to_dev_bf16(kp_host), to_dev_bf16(vp_host)
    kp_ref, vp_ref = kp_host.copy(), vp_host.copy()
    flags = guarded_flags()
    ws = guarded_workspace(SLOTS, MB)
    decoded = prefilled = 0
    for step in range(200):
        for slot in m.schedule():
            # prefill: request ids are the submission order, so the id names the prompt
            rid = m.slot_request(slot)
            prompt = REQUESTS[rid][0]
            m.set_length(slot, prompt)
            bt_all = m.block_tables()
            for layer in range(LAYERS):
                bt = bt_all[layer, slot:slot + 1]
                q = bf16(rng, (1, prompt, 32, 64))
                kc, vc = bf16(rng, (1, prompt, 8, 64)), bf16(rng, (1, prompt, 8, 64))
                qd = to_dev_bf16(q)
                out = guarded_empty(qd.shape, qd.dtype)
                binding.prefill_chunk(out, qd, to_dev_bf16(kc), to_dev_bf16(vc), kp, vp, to_dev_i32(bt),
                                      to_dev_i32(np.zeros(1, np.int32)), table, SCALE, device_flags=flags)
                q_ref = q.copy()
                ref, rc = oracle.prefill_chunk(q_ref, kc, vc, kp_ref, vp_ref, bt, np.zeros(1, np.int32), P,
                                               W.ROPE_THETA, SCALE)
                assert rc == oracle.OK
                assert_close(to_host_f64(out), ref, TOL_BF16, f"step {step} prefill slot {slot} layer {layer}")
            prefilled += 1
        lens = m.lengths()
        active = [s for s in range(SLOTS) if m.slot_request(s) >= 0 and lens[s] < m.slot_budget(s)]
        if not active and m.queued == 0 and all(m.slot_request(s) < 0 for s in range(SLOTS)):
            break
        if active:
            for s in active:
                m.set_length(s, int(lens[s]) + 1)
            bt_all = m.block_tables()
            L = m.lengths()[active].astype(np.int32)
            for layer in range(LAYERS):
                bt = np.ascontiguousarray(bt_all[layer, active])
                q = bf16(rng, (len(active), 32, 64))
                kn, vn = bf16(rng, (len(active), 8, 64)), bf16(rng, (len(active), 8, 64))
                qd = to_dev_bf16(q)
                out = guarded_empty(qd.shape, qd.dtype)
                binding.append_decode_gqa(out, qd, to_dev_bf16(kn), to_dev_bf16(vn), kp, vp, to_dev_i32(bt),
                                          to_dev_i32(L), table, SCALE, workspace=ws, device_flags=flags)
                q_ref = q.copy()
                assert oracle.append_kv_rope(q_ref, kn, vn, kp_ref, vp_ref, bt, L, P, W.ROPE_THETA) == oracle.OK
                ref, rc = oracle.decode_gqa(q_ref, kp_ref, vp_ref, bt, L, P, SCALE)
                assert rc == oracle.OK
                assert_close(to_host_f64(out), ref, TOL_BF16, f"step {step} decode layer {layer} lens {L.tolist()}")
            decoded += len(active)
        for s in range(SLOTS):  # finished: budget full
            if m.slot_request(s) >= 0 and m.lengths()[s] == m.slot_budget(s):
                m.release(s)
    else:
        pytest.fail("decode loop did not drain the queue")
    torch.cuda.synchronize()
    assert int(flags.item()) == 0
    assert prefilled == len(REQUESTS)
    assert decoded == sum(n - 1 for _, n in REQUESTS)
    assert m.free_pages == P and m.reserved_pages == 0
    # whole pools, bit for bit (V copies and rotated K rows)
    assert np.array_equal(to_host_bits(vp), vp_ref)
    assert_rope_equal(to_host_bits(kp), kp_ref, "K pool")
