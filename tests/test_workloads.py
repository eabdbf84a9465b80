"""Seeded synthetic workloads: determinism, page-table structure and the geometry the pages print."""
import json
import os

import numpy as np

from paged_kv_gqa_append_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "geometry.json")


def test_geometry_matches_pages():
    g = {k: v["value"] for k, v in json.load(open(GOLDEN)).items() if not k.startswith("_")}
    assert W.NUM_Q_HEADS == g["num_q_heads"]
    assert W.HEAD_DIM == g["embedding_length"] // g["num_q_heads"]
    assert W.NUM_KV_HEADS == g["kv_dim"] // W.HEAD_DIM
    assert W.PAGE_SIZE == g["page_tokens"]
    assert W.MAX_CONTEXT == g["max_context"]
    # one token of one layer: K and V rows of KV_DIM bf16 each
    assert W.KV_BYTES_PER_TOKEN_LAYER == 2 * g["kv_dim"] * 2 == 2048
    # the decode-time K (or V) batch buffer: BATCH_SIZE x KV_DIM bf16
    assert g["batch_size"] * g["kv_dim"] * 2 == g["decode_kv_batch_buffer_bytes"]
    # tiny-vllm's 2 GB pool over 65536 blocks: 32 KiB per block = 16 tokens of K+V
    assert g["kv_cache_bytes_tinyvllm"] // g["free_blocks_tinyvllm"] == W.PAGE_SIZE * W.KV_BYTES_PER_TOKEN_LAYER
    # samir-vllm's 128 MiB default pool: 4096 pages of 16 tokens
    assert g["default_pool_mib"] * 2 ** 20 // (W.PAGE_SIZE * W.KV_BYTES_PER_TOKEN_LAYER) == 4096
    assert g["block_table_unassigned"] == -1


def test_cases_are_deterministic():
    a, b = W.batch8_decode(), W.batch8_decode()
    for f in ("context_lens", "block_tables", "q", "k_new", "v_new", "k_pool", "v_pool"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f
    assert not np.array_equal(W.batch8_decode(seed=5).q, a.q)


def _check_tables(bt, lens, num_pages):
    need = W.pages_needed(lens)
    ids = []
    for layer in range(bt.shape[0]):
        for s, n in enumerate(need):
            row = bt[layer, s]
            assert np.all(row[:n] >= 0) and np.all(row[:n] < num_pages)
            assert np.all(row[n:] == -1)
            ids.append(row[:n])
    ids = np.concatenate(ids)
    assert len(np.unique(ids)) == len(ids), "a physical page is shared"


def test_tiny_and_batch8_tables():
    t = W.tiny_decode()
    assert t.num_pages == 64 and list(t.context_lens) == [64]
    _check_tables(t.block_tables, t.context_lens, 64)
    b = W.batch8_decode()
    assert b.num_pages == 4096 and b.k_pool.nbytes + b.v_pool.nbytes == 128 * 2 ** 20
    assert b.context_lens.min() >= 1 and b.context_lens.max() <= 2048
    _check_tables(b.block_tables, b.context_lens, 4096)


def test_poison_marks_only_unused_slots():
    c = W.make_decode_case("p", 1, [17, 3], num_pages=8)
    used = np.zeros((8, 16), bool)
    p, t = W.used_slots(c.block_tables[0], c.context_lens)
    used[p, t] = True
    nan = np.isnan(W.bf16_bits_to_f32(c.k_pool)).all(axis=(1, 3))
    assert np.array_equal(nan, ~used)


def test_batch64_and_batch256_specs():
    s = W.batch64_spec(num_layers=16)
    assert s.num_pages == 64 * 128 * 16 and s.kv_bytes() == 4 * 2 ** 30
    _check_tables(s.block_tables, s.context_lens, s.num_pages)
    r = W.batch256_spec()
    _check_tables(r.block_tables, r.context_lens, r.num_pages)
    assert r.context_lens.min() >= 1 and r.context_lens.max() <= 2048
    # fragmentation: consecutive blocks of a sequence are rarely consecutive pages
    row = r.block_tables[0][np.argmax(r.context_lens)]
    steps = np.diff(row[row >= 0])
    assert np.mean(steps == 1) < 0.5 and np.any(steps < 0)
    n_used = int(r.context_lens.sum()) * r.num_layers
    assert abs(len(r.outlier_slots) - 0.01 * n_used) <= 1
