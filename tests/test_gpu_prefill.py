"""GPU parity of pa_prefill_chunk (append the chunk, then causal paged attention on MFMA).

Bar: appended K rows, rotated q, V rows and every other pool byte bit-exact
(the device rotates with the oracle's fp64 operations); attention outputs within
1e-2 + 1e-2|ref| (bf16) or 2e-3 + 2e-3|ref| (fp32) of the fp64 oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from _gpu_helpers import (TOL_BF16, TOL_FP32, assert_close, assert_rope_equal, dev, rope, to_dev_bf16,
                          to_dev_i32, to_host_bits, to_host_f64)
from _gpu_helpers import guarded_empty, guarded_full, guarded_flags
from paged_kv_gqa_append_amd import binding
from paged_kv_gqa_append_amd import workloads as W

pytestmark = pytest.mark.gpu


class DevPrefill:
    def __init__(self, c: W.PrefillCase):
        self.c = c
        self.q = to_dev_bf16(c.q)
        self.kc = to_dev_bf16(c.k_chunk)
        self.vc = to_dev_bf16(c.v_chunk)
        self.kp = to_dev_bf16(c.k_pool)
        self.vp = to_dev_bf16(c.v_pool)
        self.bt = to_dev_i32(c.block_tables)
        self.prefix = to_dev_i32(c.prefix_lens)
        self.flags = guarded_flags()

    def run(self, out_dtype=torch.bfloat16, table=None, alias=False):
        table = rope(max_pos=4200) if table is None else table
        out = self.q if alias else guarded_empty(self.q.shape, out_dtype)
        binding.prefill_chunk(out, self.q, self.kc, self.vc, self.kp, self.vp, self.bt, self.prefix, table,
                              self.c.scale, device_flags=self.flags)
        torch.cuda.synchronize()
        return out


def oracle_all(c):
    q, kp, vp = c.q.copy(), c.k_pool.copy(), c.v_pool.copy()
    out, rc = oracle.prefill_chunk(q, c.k_chunk, c.v_chunk, kp, vp, c.block_tables, c.prefix_lens, c.num_pages,
                                   c.theta, c.scale)
    assert rc == oracle.OK
    return out, q, kp, vp



SMALL = {
    "fresh": ([0, 0], 40),
    "ragged": ([5, 16, 33], 37),
    "one_token": ([0, 7, 100], 1),
    "long_prefix": ([300, 1000], 70),
}


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_prefill_small_against_oracle(name, out_dtype):
    prefix, chunk = SMALL[name]
    c = W.make_prefill_case(name, 70 + chunk, prefix, chunk, poison=True)
    print(f"prefill case={name} prefix={prefix} chunk={chunk} out={out_dtype}", flush=True)
    d = DevPrefill(c)
    got = to_host_f64(d.run(out_dtype))
    ref, oq, okp, ovp = oracle_all(c)
    assert int(d.flags.item()) == 0
    assert_close(got, ref, TOL_BF16 if out_dtype == torch.bfloat16 else TOL_FP32, name)
    # the append part: pools and rotated q
    gk, gv, gq = to_host_bits(d.kp), to_host_bits(d.vp), to_host_bits(d.q)
    assert np.array_equal(gv, ovp)
    assert_rope_equal(gk, okp, "K pool")
    diff_slots = np.any(gk != okp, axis=(1, 3))
    written = np.zeros_like(diff_slots)
    for s, P0 in enumerate(c.prefix_lens):
        for i in range(chunk):
            t = P0 + i
            written[c.block_tables[s, t // 16], t % 16] = True
    assert not np.any(diff_slots & ~written), "bytes outside the chunk's slots differ"
    assert_rope_equal(gq, oq, "rotated q")


def test_prefill_output_may_alias_q():
    c = W.make_prefill_case("alias", 80, [3, 40], 45, poison=True)
    sep = to_host_bits(DevPrefill(c).run(torch.bfloat16))
    d = DevPrefill(c)
    out = d.run(alias=True)
    assert out.data_ptr() == d.q.data_ptr()
    assert np.array_equal(to_host_bits(out), sep)


def test_prefill_chunk_of_one_matches_decode():
    c = W.make_prefill_case("one", 81, [0, 17, 300], 1, poison=True)
    got = to_host_f64(DevPrefill(c).run(torch.float32))[:, 0]
    q, kp, vp = c.q[:, 0].copy(), c.k_pool.copy(), c.v_pool.copy()
    lens = (c.prefix_lens + 1).astype(np.int32)
    assert oracle.append_kv_rope(q, c.k_chunk[:, 0], c.v_chunk[:, 0], kp, vp, c.block_tables, lens, c.num_pages,
                                 c.theta) == oracle.OK
    ref, rc = oracle.decode_gqa(q, kp, vp, c.block_tables, lens, c.num_pages, c.scale)
    assert rc == oracle.OK
    assert_close(got, ref, TOL_FP32, "chunk of one")


def test_prefill_config_full_size_all_rows():
    """4 sequences x (1536 cached + 512 chunk), in the benchmark's launch: every row of every
    sequence against the oracle's prefill, and the pools and rotated q bit for bit."""
    c = W.prefill_config()
    d = DevPrefill(c)
    got = to_host_f64(d.run(torch.bfloat16))
    assert int(d.flags.item()) == 0
    ref, oq, okp, ovp = oracle_all(c)
    assert_close(got, ref, TOL_BF16, "prefill config, all rows")
    assert_rope_equal(to_host_bits(d.kp), okp, "K pool")
    assert np.array_equal(to_host_bits(d.vp), ovp)
    assert_rope_equal(to_host_bits(d.q), oq, "rotated q")


def _all_rows_case(c, table=None):
    """Run one case on the GPU and return it with the oracle's output, rotated q and pools."""
    d = DevPrefill(c)
    got = to_host_f64(d.run(torch.bfloat16, table=table))
    assert int(d.flags.item()) == 0
    ref, oq, okp, ovp = oracle_all(c)
    return d, got, ref, oq, okp, ovp


@pytest.mark.parametrize("prefix,chunk", [([0, 3, 60], 512), ([5, 0, 17, 40, 2], 448)])
def test_prefill_workgroup_turns(prefix, chunk):
    """Workgroup ids are dealt to an XCD's 32 CUs in turns, every second turn in reverse order.
    Grids with 48 workgroups per XCD (3 sequences x 16 tiles: the reversed turn only half full) and
    70 (5 x 14: three turns, the last one short) must still cover every (sequence, KV head, tile)
    once: every row against the oracle, pools and rotated q bit for bit."""
    c = W.make_prefill_case("turns", 83 + len(prefix), prefix, chunk, poison=True)
    d, got, ref, oq, okp, ovp = _all_rows_case(c)
    assert_close(got, ref, TOL_BF16, f"{len(prefix)} x {chunk}, all rows")
    assert_rope_equal(to_host_bits(d.kp), okp, "K pool")
    assert np.array_equal(to_host_bits(d.vp), ovp)
    assert_rope_equal(to_host_bits(d.q), oq, "rotated q")


def test_prefill_past_4096_keys():
    """Contexts of 4,548 and 6,048 keys: a key half then has more than 64 blocks, whose page ids
    the kernel looks up in LDS instead of keeping them in lanes, and a sequence has more pages
    than the workgroup has threads (two block-table entries per thread in validation)."""
    c = W.make_prefill_case("long", 84, [4500, 6000, 100], 48, poison=True)
    assert c.max_blocks > 256
    d, got, ref, oq, okp, ovp = _all_rows_case(c, table=rope(max_pos=6200))
    assert_close(got, ref, TOL_BF16, "contexts past 4096 keys")
    assert_rope_equal(to_host_bits(d.kp), okp, "K pool")
    assert np.array_equal(to_host_bits(d.vp), ovp)
    assert_rope_equal(to_host_bits(d.q), oq, "rotated q")


def test_prefill_batch_invariance():
    """A sequence's rows come out bit for bit the same alone and inside a batch (the workgroup order
    changes with the grid; the arithmetic of a tile does not)."""
    c = W.make_prefill_case("inv", 85, [7, 300, 40, 1030, 0], 70, poison=True)
    batch = to_host_bits(DevPrefill(c).run(torch.float32))
    for s in range(c.num_seqs):
        one = W.PrefillCase(name="one", num_seqs=1, chunk_len=c.chunk_len, max_blocks=c.max_blocks,
                            num_pages=c.num_pages, prefix_lens=c.prefix_lens[s:s + 1].copy(),
                            block_tables=c.block_tables[s:s + 1].copy(), q=c.q[s:s + 1].copy(),
                            k_chunk=c.k_chunk[s:s + 1].copy(), v_chunk=c.v_chunk[s:s + 1].copy(),
                            k_pool=c.k_pool, v_pool=c.v_pool)
        alone = to_host_bits(DevPrefill(one).run(torch.float32))
        assert np.array_equal(alone[0], batch[s]), f"sequence {s}"


def test_prefill_device_errors():
    c = W.make_prefill_case("err", 82, [10, 20, 30], 16, poison=True)
    d = DevPrefill(c)
    prefix = c.prefix_lens.copy()
    prefix[0] = -1                   # bad prefix length
    bt = c.block_tables.copy()
    bt[2, 1] = c.num_pages + 5       # bad page among sequence 2's used pages
    d.prefix, d.bt = to_dev_i32(prefix), to_dev_i32(bt)
    out = guarded_full(d.q.shape, 3.0, torch.float32)
    binding.prefill_chunk(out, d.q, d.kc, d.vc, d.kp, d.vp, d.bt, d.prefix, rope(max_pos=4200), c.scale,
                          device_flags=d.flags)
    torch.cuda.synchronize()
    assert int(d.flags.item()) == binding.PA_DEVERR_CONTEXT_LEN | binding.PA_DEVERR_PAGE_ID
    got = to_host_f64(out)
    assert np.all(got[0] == 0) and np.all(got[2] == 0)
    ref, _, _, _ = oracle_all(W.PrefillCase(name="one", num_seqs=1, chunk_len=16, max_blocks=c.max_blocks,
                                            num_pages=c.num_pages, prefix_lens=c.prefix_lens[1:2].copy(),
                                            block_tables=c.block_tables[1:2].copy(), q=c.q[1:2].copy(),
                                            k_chunk=c.k_chunk[1:2].copy(), v_chunk=c.v_chunk[1:2].copy(),
                                            k_pool=c.k_pool, v_pool=c.v_pool))
    assert_close(got[1], ref[0], TOL_FP32, "healthy sequence")
