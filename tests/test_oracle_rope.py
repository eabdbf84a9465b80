"""Pins for the oracle's rotary embedding and decode-time KV append.

Reading (the pages never spell RoPE out; the tiny-vllm chapter only says a
frequency table is built at init, section "What else is set up in the
initialization block", and the samir-vllm article, section "Gestion de la KV
cache ...", says each new token is appended at its absolute RoPE position):
rotate-half pairs (i, i+32), w_i = theta^(-2i/64), theta = 500000, no
frequency scaling, position = L - 1.
"""
import numpy as np
import pytest
import torch

from paged_kv_gqa_append_amd import workloads as W

THETA = 500000.0


def rand_head(rng, scale=1.0):
    return W.f32_to_bf16_bits(rng.standard_normal(64).astype(np.float32) * scale)


def test_pos0_is_identity(oracle_lib):
    rng = np.random.default_rng(0)
    for _ in range(20):
        x = rand_head(rng)
        y = oracle_lib.rope_head(x, 0, THETA)
        assert np.array_equal(y, W.bf16_bits_to_f32(x).astype(np.float64))


@pytest.mark.parametrize("pos", [1, 7, 63, 1000, 2047, 4095])
def test_matches_complex_multiplication(oracle_lib, pos):
    rng = np.random.default_rng(pos)
    x = rand_head(rng)
    xf = W.bf16_bits_to_f32(x).astype(np.float64)
    i = np.arange(32)
    w = THETA ** (-2.0 * i / 64.0)
    z = (xf[:32] + 1j * xf[32:]) * np.exp(1j * pos * w)
    y = oracle_lib.rope_head(x, pos, THETA)
    np.testing.assert_allclose(y[:32], z.real, rtol=0, atol=1e-12)
    np.testing.assert_allclose(y[32:], z.imag, rtol=0, atol=1e-12)


def test_matches_hf_llama_rotate_half(oracle_lib):
    """Hugging Face's Llama rotary routine (float32 angles) agrees to its own precision."""
    from transformers import LlamaConfig
    from transformers.models.llama.modeling_llama import LlamaRotaryEmbedding, apply_rotary_pos_emb

    cfg = LlamaConfig(hidden_size=2048, num_attention_heads=32, num_key_value_heads=8, head_dim=64,
                      max_position_embeddings=4096,
                      rope_parameters={"rope_type": "default", "rope_theta": THETA})
    emb = LlamaRotaryEmbedding(cfg)
    rng = np.random.default_rng(5)
    pos = np.array([0, 1, 2, 15, 16, 17, 255, 1000, 2046, 2047])
    x = np.stack([rand_head(rng) for _ in pos])
    xt = torch.from_numpy(W.bf16_bits_to_f32(x).astype(np.float64))[None, None]  # [1,1,n,64]
    cos, sin = emb(xt.float(), torch.from_numpy(pos)[None])
    qr, _ = apply_rotary_pos_emb(xt, xt, cos.double(), sin.double(), unsqueeze_dim=1)
    ref = qr[0, 0].numpy()
    got = np.stack([oracle_lib.rope_head(x[k], int(p), THETA) for k, p in enumerate(pos)])
    # HF evaluates the angle in float32: error <= pos * 2^-24 rad per pair
    np.testing.assert_allclose(got, ref, rtol=0, atol=2e-3)
    # and the gross structure exactly: with the angle from float32 inv_freq, errors vanish at pos 0
    np.testing.assert_allclose(got[0], ref[0], rtol=0, atol=0)


def test_pair_norm_and_relative_position(oracle_lib):
    rng = np.random.default_rng(9)
    q, k = rand_head(rng), rand_head(rng)
    qf = W.bf16_bits_to_f32(q).astype(np.float64)
    for pos in (3, 100, 2047):
        y = oracle_lib.rope_head(q, pos, THETA)
        np.testing.assert_allclose(y[:32] ** 2 + y[32:] ** 2, qf[:32] ** 2 + qf[32:] ** 2, rtol=1e-13)
    # <R_m q, R_n k> depends on m - n only
    d = []
    for m, n in ((10, 3), (107, 100), (2047, 2040)):
        d.append(float(oracle_lib.rope_head(q, m, THETA) @ oracle_lib.rope_head(k, n, THETA)))
    assert abs(d[0] - d[1]) < 1e-9 and abs(d[0] - d[2]) < 1e-9
    # pair 0 has w_0 = 1: it turns by exactly pos radians
    y = oracle_lib.rope_head(q, 5, THETA)
    assert abs(y[0] - (qf[0] * np.cos(5.0) - qf[32] * np.sin(5.0))) < 1e-15


def _append_case(seed=0, lens=(1, 15, 16, 17, 40), num_pages=20):
    return W.make_decode_case("append", seed, list(lens), num_layers=1, num_pages=num_pages, poison=True)


def test_append_writes_exactly_one_slot_per_sequence(oracle_lib):
    c = _append_case()
    kp, vp, q = c.k_pool.copy(), c.v_pool.copy(), c.q[0].copy()
    rc = oracle_lib.append_kv_rope(q, c.k_new[0], c.v_new[0], kp, vp, c.block_tables[0], c.context_lens,
                                   c.num_pages, THETA)
    assert rc == oracle_lib.OK
    changed_k = np.zeros((c.num_pages, 16), bool)
    changed_k |= np.any(kp.view(np.int16) != c.k_pool.view(np.int16), axis=(1, 3))
    changed_v = np.any(vp.view(np.int16) != c.v_pool.view(np.int16), axis=(1, 3))
    expect = np.zeros_like(changed_k)
    for s, L in enumerate(c.context_lens):
        pos = int(L) - 1
        page, slot = c.block_tables[0, s, pos // 16], pos % 16
        expect[page, slot] = True
        # V: exact copy; K: one-step bf16 of the fp64 rotation; q rotated in place
        assert np.array_equal(vp[page, :, slot, :], c.v_new[0, s])
        for j in range(8):
            ref = np.array([oracle_lib.f64_to_bf16(v) for v in oracle_lib.rope_head(c.k_new[0, s, j], pos, THETA)],
                           dtype=np.uint16)
            assert np.array_equal(kp[page, j, slot, :], ref)
        for h in range(32):
            ref = np.array([oracle_lib.f64_to_bf16(v) for v in oracle_lib.rope_head(c.q[0, s, h], pos, THETA)],
                           dtype=np.uint16)
            assert np.array_equal(q[s, h], ref)
    # appended slots were NaN-poisoned before, so every one of them changed
    assert np.array_equal(changed_k, expect)
    assert np.array_equal(changed_v, expect)


def test_append_null_q_and_errors(oracle_lib):
    c = _append_case()
    kp, vp = c.k_pool.copy(), c.v_pool.copy()
    assert oracle_lib.append_kv_rope(None, c.k_new[0], c.v_new[0], kp, vp, c.block_tables[0], c.context_lens,
                                     c.num_pages, THETA) == oracle_lib.OK
    bad = c.context_lens.copy()
    bad[0] = 0
    assert oracle_lib.append_kv_rope(None, c.k_new[0], c.v_new[0], kp, vp, c.block_tables[0], bad,
                                     c.num_pages, THETA) == oracle_lib.BAD_LEN
    bt = c.block_tables[0].copy()
    L = int(c.context_lens[1])
    bt[1, (L - 1) // 16] = c.num_pages  # out of range
    assert oracle_lib.append_kv_rope(None, c.k_new[0], c.v_new[0], kp, vp, bt, c.context_lens,
                                     c.num_pages, THETA) == oracle_lib.BAD_PAGE
