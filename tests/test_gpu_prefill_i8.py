"""GPU parity of pa_prefill_chunk_i8 (quantise the chunk into INT8 pages, then causal
attention over them) against the oracle's INT8 prefill.

Bar: every pool byte bit-exact after the append (codes and scales are decisions the
format fixes in binary32), rotated q bit-exact (the oracle's fp64 operations), and
attention outputs within 1e-2 + 1e-2|ref| (bf16 out) or 2e-3 + 2e-3|ref| (fp32 out) of
the fp64 oracle over the values code * scale, as for the INT8 decode.
"""
import numpy as np
import pytest
import torch

import oracle
from _gpu_helpers import (TOL_BF16, TOL_FP32, assert_close, assert_rope_equal, guarded_empty, guarded_flags, rope,
                          to_dev_bf16, to_dev_i32, to_dev_u8, to_host_bits, to_host_f64)
from paged_kv_gqa_append_amd import binding
from paged_kv_gqa_append_amd import workloads as W

pytestmark = pytest.mark.gpu


class DevPrefillI8:
    def __init__(self, c: W.PrefillCase, pool_i8, prefix=None, bt=None):
        self.c = c
        self.q = to_dev_bf16(c.q)
        self.kc = to_dev_bf16(c.k_chunk)
        self.vc = to_dev_bf16(c.v_chunk)
        self.pool = to_dev_u8(pool_i8)
        self.bt = to_dev_i32(c.block_tables if bt is None else bt)
        self.prefix = to_dev_i32(c.prefix_lens if prefix is None else prefix)
        self.flags = guarded_flags()

    def run(self, out_dtype=torch.bfloat16, alias=False):
        out = self.q if alias else guarded_empty(self.q.shape, out_dtype)
        binding.prefill_chunk_i8(out, self.q, self.kc, self.vc, self.pool, self.bt, self.prefix, rope(max_pos=4200),
                                 self.c.scale, device_flags=self.flags)
        torch.cuda.synchronize()
        return out


def oracle_rows(c, pool_i8, rows=None):
    """The oracle's INT8 prefill (appending every chunk token), its output for `rows` (all when
    None), and the q and pool it leaves."""
    q, pool = c.q.copy(), pool_i8.copy()
    if rows is None:
        out, rc = oracle.prefill_chunk_i8(q, c.k_chunk, c.v_chunk, pool, c.block_tables, c.prefix_lens,
                                          c.num_pages, c.theta, c.scale)
        assert rc == oracle.OK
        return out, q, pool
    for i in range(c.chunk_len):  # the append only (the composition's first half)
        qi = np.ascontiguousarray(q[:, i])
        assert oracle.append_kv_rope_i8(qi, c.k_chunk[:, i], c.v_chunk[:, i], pool, c.block_tables,
                                        (c.prefix_lens + i + 1).astype(np.int32), c.num_pages, c.theta) == oracle.OK
        q[:, i] = qi
    out = np.zeros((c.num_seqs, len(rows), 32, 64))
    for k, i in enumerate(rows):
        o, rc = oracle.decode_gqa_i8(q[:, i], pool, c.block_tables, (c.prefix_lens + i + 1).astype(np.int32),
                                     c.num_pages, c.scale)
        assert rc == oracle.OK
        out[:, k] = o
    return out, q, pool


SMALL = {
    "fresh": ([0, 0], 40),
    "ragged": ([5, 16, 33], 37),
    "one_token": ([0, 7, 100], 1),
    "long_prefix": ([300, 1000], 70),
}


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_prefill_i8_against_oracle(name, out_dtype):
    prefix, chunk = SMALL[name]
    c = W.make_prefill_case(name, 170 + chunk, prefix, chunk, poison=True)
    print(f"i8 prefill case={name} prefix={prefix} chunk={chunk} out={out_dtype}", flush=True)
    pool = oracle.quantize_pages_i8(c.k_pool, c.v_pool)
    d = DevPrefillI8(c, pool)
    got = to_host_f64(d.run(out_dtype))
    assert int(d.flags.item()) == 0
    ref, oq, opool = oracle_rows(c, pool)
    assert np.array_equal(d.pool.cpu().numpy(), opool), "INT8 pool after the append"
    assert_rope_equal(to_host_bits(d.q), oq, "rotated q")
    assert_close(got, ref, TOL_BF16 if out_dtype == torch.bfloat16 else TOL_FP32, name)


def test_prefill_i8_output_may_alias_q():
    c = W.make_prefill_case("alias8", 180, [3, 40], 45, poison=True)
    pool = oracle.quantize_pages_i8(c.k_pool, c.v_pool)
    sep = to_host_bits(DevPrefillI8(c, pool).run(torch.bfloat16))
    d = DevPrefillI8(c, pool)
    out = d.run(alias=True)
    assert out.data_ptr() == d.q.data_ptr()
    assert np.array_equal(to_host_bits(out), sep)


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_prefill_i8_outliers_and_wide_values(out_dtype):
    """Rows scaled x20 (1 % of the pool) and a chunk whose V rows reach 1e4: the scales and the
    lazy V exponent carry them; outputs within the fp32 bar, or the bf16 one for bf16 output
    (where pairs of pages with a V scale above 1/8 take the lo weight halves and the rest not)."""
    c = W.make_prefill_case("wide8", 181, [64, 200], 50, poison=True)
    rng = np.random.default_rng(5)
    kp = W.bf16_bits_to_f32(c.k_pool).copy()
    rows = rng.random(kp.shape[:3]) < 0.01
    kp[rows] *= 20
    c.k_pool = W.f32_to_bf16_bits(kp)
    vc = W.bf16_bits_to_f32(c.v_chunk).copy()
    vc[:, ::7] *= 1e4
    c.v_chunk = W.f32_to_bf16_bits(vc)
    pool = oracle.quantize_pages_i8(c.k_pool, c.v_pool)
    d = DevPrefillI8(c, pool)
    got = to_host_f64(d.run(out_dtype))
    ref, _, opool = oracle_rows(c, pool)
    assert np.array_equal(d.pool.cpu().numpy(), opool)
    assert_close(got, ref, TOL_FP32 if out_dtype == torch.float32 else TOL_BF16, "outliers and wide V")


def test_prefill_i8_device_errors():
    """A bad prefix and a bad page id in the used range: those sequences' rows are zero and the
    flags set; the good sequence is appended and attended as alone."""
    c = W.make_prefill_case("err8", 182, [10, 20, 5], 30, poison=True)
    pool = oracle.quantize_pages_i8(c.k_pool, c.v_pool)
    prefix = c.prefix_lens.copy()
    bt = c.block_tables.copy()
    prefix[0] = -1
    bt[1, 0] = c.num_pages
    d = DevPrefillI8(c, pool, prefix=prefix, bt=bt)
    got = to_host_f64(d.run(torch.float32))
    assert int(d.flags.item()) == binding.PA_DEVERR_CONTEXT_LEN | binding.PA_DEVERR_PAGE_ID
    assert np.all(got[0] == 0) and np.all(got[1] == 0)
    sub = W.PrefillCase(**{**c.__dict__})
    for k in ("q", "k_chunk", "v_chunk", "block_tables", "prefix_lens"):
        setattr(sub, k, getattr(c, k)[2:3].copy())
    sub.num_seqs = 1
    ref, _, _ = oracle_rows(sub, pool)
    assert_close(got[2:3], ref, TOL_FP32, "good sequence beside bad ones")


def test_prefill_i8_config_full_size_sampled_rows():
    """4 sequences x (1536 cached + 512 chunk), the benchmark's launch: the whole pool and every
    rotated q row bit for bit; the outputs of 64 rows per sequence (every 8th, the first and the
    last included) against the oracle."""
    c = W.prefill_config()
    pool = oracle.quantize_pages_i8(c.k_pool, c.v_pool)
    d = DevPrefillI8(c, pool)
    got = to_host_f64(d.run(torch.bfloat16))
    assert int(d.flags.item()) == 0
    rows = sorted(set(range(0, c.chunk_len, 8)) | {c.chunk_len - 1})
    ref, oq, opool = oracle_rows(c, pool, rows)
    assert np.array_equal(d.pool.cpu().numpy(), opool)
    assert_rope_equal(to_host_bits(d.q), oq, "rotated q")
    assert_close(got[:, rows], ref, TOL_BF16, "prefill config, sampled rows")
