"""Pins for the oracle's chunked prefill (append the chunk, then causal paged attention).

The chunked form follows TinyLoop's "prefill_chunk and scratch residency"
section (prompt processed in row chunks); the paged storage follows the
samir-vllm article, section "Gestion de la KV cache ...": during prefill the
prompt's pages are filled.  Reading: causal, inclusive (a query sees its own key).
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from paged_kv_gqa_append_amd import workloads as W

THETA = 500000.0


def clone(c):
    return (c.q.copy(), c.k_pool.copy(), c.v_pool.copy())


def run(oracle_lib, c, q, kp, vp, k_chunk=None, v_chunk=None, prefix=None):
    out, rc = oracle_lib.prefill_chunk(q, c.k_chunk if k_chunk is None else k_chunk,
                                       c.v_chunk if v_chunk is None else v_chunk, kp, vp, c.block_tables,
                                       c.prefix_lens if prefix is None else prefix, c.num_pages, THETA, c.scale)
    assert rc == oracle_lib.OK
    return out


def gather(pool, bt_row, n):
    t = np.arange(n)
    return W.bf16_bits_to_f32(pool[bt_row[t // 16], :, t % 16, :]).astype(np.float64).transpose(1, 0, 2)


@pytest.mark.parametrize("prefix,chunk", [([0, 0], 40), ([5, 16], 21), ([33, 0, 70], 17)])
def test_matches_masked_sdpa(oracle_lib, prefix, chunk):
    c = W.make_prefill_case("pin", 20 + chunk, prefix, chunk, poison=True)
    q, kp, vp = clone(c)
    out = run(oracle_lib, c, q, kp, vp)
    for s, P in enumerate(c.prefix_lens):
        n = int(P) + chunk
        k = torch.from_numpy(gather(kp, c.block_tables[s], n))[None]
        v = torch.from_numpy(gather(vp, c.block_tables[s], n))[None]
        qq = torch.from_numpy(W.bf16_bits_to_f32(q[s]).astype(np.float64).transpose(1, 0, 2))[None]
        pos_q = torch.arange(chunk)[:, None] + int(P)
        mask = torch.arange(n)[None, :] <= pos_q  # causal, inclusive
        ref = F.scaled_dot_product_attention(qq, k, v, attn_mask=mask, scale=c.scale, enable_gqa=True)
        np.testing.assert_allclose(out[s], ref[0].numpy().transpose(1, 0, 2), rtol=1e-12, atol=1e-12)
        if int(P) == 0:  # textbook causal attention
            ref2 = F.scaled_dot_product_attention(qq, k, v, is_causal=True, scale=c.scale, enable_gqa=True)
            np.testing.assert_allclose(out[s], ref2[0].numpy().transpose(1, 0, 2), rtol=1e-12, atol=1e-12)


def test_chunk_rows_equal_decode(oracle_lib):
    c = W.make_prefill_case("rows", 30, [19, 48], 9, poison=True)
    q, kp, vp = clone(c)
    out = run(oracle_lib, c, q, kp, vp)
    # every chunk row i equals decode at L = prefix + i + 1 over the filled pages
    for i in range(9):
        lens = (c.prefix_lens + i + 1).astype(np.int32)
        dec, rc = oracle_lib.decode_gqa(np.ascontiguousarray(q[:, i]), kp, vp, c.block_tables, lens,
                                        c.num_pages, c.scale)
        assert rc == oracle_lib.OK
        assert np.array_equal(dec, out[:, i])


def test_chunk_of_one_equals_append_then_decode(oracle_lib):
    c = W.make_prefill_case("one", 31, [0, 7, 40], 1, poison=True)
    q, kp, vp = clone(c)
    out = run(oracle_lib, c, q, kp, vp)
    q2, kp2, vp2 = c.q[:, 0].copy(), c.k_pool.copy(), c.v_pool.copy()
    lens = (c.prefix_lens + 1).astype(np.int32)
    assert oracle_lib.append_kv_rope(q2, c.k_chunk[:, 0], c.v_chunk[:, 0], kp2, vp2, c.block_tables, lens,
                                     c.num_pages, THETA) == oracle_lib.OK
    assert np.array_equal(kp, kp2) and np.array_equal(vp, vp2) and np.array_equal(q[:, 0], q2)
    dec, rc = oracle_lib.decode_gqa(q2, kp2, vp2, c.block_tables, lens, c.num_pages, c.scale)
    assert rc == oracle_lib.OK and np.array_equal(dec, out[:, 0])


def test_two_half_chunks_equal_one(oracle_lib):
    c = W.make_prefill_case("split", 32, [3, 20], 24, poison=True)
    q, kp, vp = clone(c)
    whole = run(oracle_lib, c, q, kp, vp)
    qa = np.ascontiguousarray(c.q[:, :12])
    qb = np.ascontiguousarray(c.q[:, 12:])
    kp2, vp2 = c.k_pool.copy(), c.v_pool.copy()
    a = run(oracle_lib, c, qa, kp2, vp2, np.ascontiguousarray(c.k_chunk[:, :12]),
            np.ascontiguousarray(c.v_chunk[:, :12]))
    b = run(oracle_lib, c, qb, kp2, vp2, np.ascontiguousarray(c.k_chunk[:, 12:]),
            np.ascontiguousarray(c.v_chunk[:, 12:]), prefix=(c.prefix_lens + 12).astype(np.int32))
    assert np.array_equal(np.concatenate([a, b], axis=1), whole)
    assert np.array_equal(kp2, kp) and np.array_equal(vp2, vp)
