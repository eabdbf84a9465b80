"""Pins of the oracle's chunked prefill into INT8 pages (oracle.prefill_chunk_i8),
which is written as the INT8 append of each chunk token followed by the INT8
decode of each chunk row.  Two checks from outside that composition:

- its outputs equal torch's fp64 causal scaled-dot-product attention over the
  values code * scale read back from the pool it leaves (the tile layout read
  independently, as in test_oracle_i8), with q as it leaves it;
- the pool and q it leaves equal those of the bf16 oracle prefill (pinned in
  test_oracle_prefill) with the appended rows then quantised by the oracle's
  page quantiser (pinned in test_oracle_i8): the same rotation, rounding and
  quantisation, in either order."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from paged_kv_gqa_append_amd import workloads as W
from test_oracle_i8 import read_row


def make_case(seed, prefixes, C, mb):
    rng = np.random.default_rng(seed)
    B = len(prefixes)
    P = B * mb + 2
    bt = rng.permutation(P)[:B * mb].astype(np.int32).reshape(B, mb)
    kp = W.f32_to_bf16_bits(rng.standard_normal((P, 8, 16, 64)).astype(np.float32))
    vp = W.f32_to_bf16_bits(rng.standard_normal((P, 8, 16, 64)).astype(np.float32))
    q = W.f32_to_bf16_bits(rng.standard_normal((B, C, 32, 64)).astype(np.float32))
    kc = W.f32_to_bf16_bits(rng.standard_normal((B, C, 8, 64)).astype(np.float32))
    vc = W.f32_to_bf16_bits(rng.standard_normal((B, C, 8, 64)).astype(np.float32))
    return np.array(prefixes, np.int32), P, bt, kp, vp, q, kc, vc


@pytest.mark.parametrize("prefixes,C", [([0, 17, 40], 20), ([3], 33)])
def test_matches_causal_sdpa_on_the_pool(prefixes, C):
    pl, P, bt, kp, vp, q, kc, vc = make_case(7 + C, prefixes, C, 6)
    pool = oracle.quantize_pages_i8(kp, vp)
    q = q.copy()
    out, rc = oracle.prefill_chunk_i8(q, kc, vc, pool, bt, pl, P, W.ROPE_THETA, 0.125)
    assert rc == oracle.OK
    for s, pre in enumerate(prefixes):
        n = pre + C
        k = np.zeros((8, n, 64))
        v = np.zeros((8, n, 64))
        for t in range(n):
            for j in range(8):
                k[j, t] = read_row(pool, bt[s, t // 16], j, t % 16, "k")[0]
                v[j, t] = read_row(pool, bt[s, t // 16], j, t % 16, "v")[0]
        qq = torch.from_numpy(W.bf16_bits_to_f32(q[s]).astype(np.float64).transpose(1, 0, 2))[None]  # [1][32][C][64]
        mask = torch.from_numpy(np.arange(n)[None, :] <= (pre + np.arange(C))[:, None])
        ref = F.scaled_dot_product_attention(qq, torch.from_numpy(k)[None], torch.from_numpy(v)[None],
                                             attn_mask=mask, scale=0.125, enable_gqa=True)[0].numpy()
        assert np.abs(out[s] - ref.transpose(1, 0, 2)).max() < 1e-12


def test_append_equals_bf16_prefill_then_quantiser():
    pl, P, bt, kp, vp, q, kc, vc = make_case(31, [5, 0, 30], 24, 5)
    pool = oracle.quantize_pages_i8(kp, vp)
    q8 = q.copy()
    _, rc = oracle.prefill_chunk_i8(q8, kc, vc, pool, bt, pl, P, W.ROPE_THETA, 0.125)
    assert rc == oracle.OK
    kb, vb, qb = kp.copy(), vp.copy(), q.copy()
    _, rc = oracle.prefill_chunk(qb, kc, vc, kb, vb, bt, pl, P, W.ROPE_THETA, 0.125)
    assert rc == oracle.OK
    assert np.array_equal(q8, qb), "rotated q differs"
    assert np.array_equal(pool, oracle.quantize_pages_i8(kb, vb)), "pool differs"


def test_bad_sequence_leaves_the_others():
    """A sequence with a bad prefix is not appended and reports BAD_LEN; the others are unchanged
    by its presence."""
    pl, P, bt, kp, vp, q, kc, vc = make_case(41, [4, 9], 10, 4)
    pool = oracle.quantize_pages_i8(kp, vp)
    qa = q.copy()
    good, rc = oracle.prefill_chunk_i8(qa, kc, vc, pool.copy(), bt, pl, P, W.ROPE_THETA, 0.125)
    assert rc == oracle.OK
    bad_pl = pl.copy()
    bad_pl[1] = -20
    qb = q.copy()
    out, rc = oracle.prefill_chunk_i8(qb, kc, vc, pool.copy(), bt, bad_pl, P, W.ROPE_THETA, 0.125)
    assert rc != oracle.OK
    assert np.array_equal(out[0], good[0]) and np.array_equal(qb[0], qa[0])
