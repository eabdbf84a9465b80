"""Pins for the oracle's INT8 K/V pages (quantiser, tile layout, append, decode).

The pages name INT8 K/V as a KV-cache storage mode (TinyLoop "Lifecycle and
Memory Model", section "Per-request / handle-owned memory") and give no rule;
the reading taken is one symmetric fp32 scale per (token, KV head) row:
scale = max|x| / 127, code = round-half-even(x / scale), decided in binary32.

* hand-checkable rows with exact scales and ties (tests/golden/i8_quant_rows.json);
* an exact-rational quantiser (fractions, binary32 rounding written out) on
  random rows, outliers and tiny values: every code and scale must agree;
* the dequantisation error bound |code*scale - x| <= scale/2 (plus the binary32
  rounding of x/scale) and max |code| = 127;
* the tile layout: the header's byte formula is a bijection onto the 2176
  bytes; rows appended by the oracle read back at those positions, nothing
  else in the pool changes;
* decode: torch's fp64 SDPA on the dequantised, gathered K/V; closed forms
  (one token -> its V, identical V rows -> that V).
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from paged_kv_gqa_append_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "i8_quant_rows.json")
TILE = 2176


def f32_round(fr: Fraction) -> Fraction:
    """Exact round-to-nearest-even of a rational to binary32 (finite range)."""
    if fr == 0:
        return Fraction(0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    spacing = Fraction(2) ** (max(e, -126) - 23)
    n = a / spacing
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * spacing


def rne_int(fr: Fraction) -> int:
    fl = fr.numerator // fr.denominator
    rem = fr - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return fl


def exact_quantise(x_f32):
    xs = [Fraction(float(v)) for v in x_f32]
    amax = max(abs(v) for v in xs)
    scale = f32_round(amax / 127)
    if scale == 0:
        return np.zeros(64, np.int64), 0.0
    codes = [max(-127, min(127, rne_int(f32_round(v / scale)))) for v in xs]
    return np.array(codes), float(scale)


def row(values):
    x = np.zeros(64, np.float32)
    x[:len(values)] = values
    return W.f32_to_bf16_bits(x)


def test_golden_rows():
    g = json.load(open(GOLDEN))
    for r in g["rows"]:
        codes, sc = oracle.quantize_row_i8(row(r["x"]))
        want = np.zeros(64, np.int64)
        want[:len(r["codes"])] = r["codes"]
        assert np.array_equal(codes.astype(np.int64), want), r["why"]
        assert float(sc) == r["scale"], r["why"]


@pytest.mark.parametrize("kind", ["normal", "outlier", "tiny", "uniform"])
def test_exact_rational_quantiser(kind):
    rng = np.random.default_rng({"normal": 1, "outlier": 2, "tiny": 3, "uniform": 4}[kind])
    for _ in range(200):
        x = rng.standard_normal(64).astype(np.float32)
        if kind == "outlier":
            x[rng.integers(64)] *= 20
        elif kind == "tiny":
            x *= np.float32(1e-30)
        elif kind == "uniform":
            x = rng.uniform(-1, 1, 64).astype(np.float32)
        bits = W.f32_to_bf16_bits(x)
        codes, sc = oracle.quantize_row_i8(bits)
        want_codes, want_sc = exact_quantise(W.bf16_bits_to_f32(bits))
        assert float(sc) == want_sc
        assert np.array_equal(codes.astype(np.int64), want_codes)


def test_error_bound_and_range():
    rng = np.random.default_rng(5)
    for _ in range(300):
        bits = W.f32_to_bf16_bits((rng.standard_normal(64) * rng.uniform(0.01, 50)).astype(np.float32))
        x = W.bf16_bits_to_f32(bits).astype(np.float64)
        codes, sc = oracle.quantize_row_i8(bits)
        assert np.abs(codes.astype(np.int64)).max() == 127      # the row's max maps to +-127
        err = np.abs(codes.astype(np.float64) * float(sc) - x)
        # half a step, plus the binary32 rounding of the quotient x/scale
        # (|x/scale| <= 127, relative error 2^-24) that decides the code
        assert err.max() <= float(sc) * (0.5 + 128 * 2.0 ** -24)


def k_pos(t, d):
    """Byte of K element d of token t in a 2176-byte tile (include/pa.h)."""
    return (((d % 32) // 8) * 16 + t) * 16 + (d // 32) * 8 + d % 8


def v_pos(t, d):
    """Byte of V element d of token t in a tile (include/pa.h)."""
    return 1024 + ((t // 4) * 16 + d % 16) * 16 + (d // 16) * 4 + t % 4


def scale_pos(t, which):
    return (2048 if which == "k" else 2112) + 4 * t


def read_row(pool, page, head, t, which):
    tile = pool[page, head]
    pos = k_pos if which == "k" else v_pos
    codes = np.array([tile[pos(t, d)] for d in range(64)], np.uint8).view(np.int8)
    sc = tile[scale_pos(t, which):][:4].view(np.float32)[0]
    return codes.astype(np.float64) * float(sc), codes, sc


def test_layout_is_a_bijection():
    """Every code byte and scale slot of a tile belongs to exactly one (row, element)."""
    seen = {}
    for t in range(16):
        for d in range(64):
            for which, pos in (("k", k_pos), ("v", v_pos)):
                b = pos(t, d)
                assert b not in seen, (which, t, d, seen.get(b))
                seen[b] = (which, t, d)
        for which in ("k", "v"):
            for b in range(scale_pos(t, which), scale_pos(t, which) + 4):
                assert b not in seen
                seen[b] = (which, t, "scale")
    assert sorted(seen) == list(range(TILE))


def test_layout_and_append_touch_only_the_row():
    """16 tokens appended one by one into a 2-page pool land where the header
    formula says, as the exact quantisation of their rows (V as given, K after
    the oracle's RoPE + bf16 rounding, both pinned elsewhere); every other
    byte keeps its value."""
    rng = np.random.default_rng(11)
    P = 2
    pool = rng.integers(0, 256, (P, 8, TILE), dtype=np.uint8)
    bt = np.array([[1, 0]], np.int32)
    for pos in range(20):
        before = pool.copy()
        kn = W.f32_to_bf16_bits(rng.standard_normal((1, 8, 64)).astype(np.float32))
        vn = W.f32_to_bf16_bits(rng.standard_normal((1, 8, 64)).astype(np.float32))
        assert oracle.append_kv_rope_i8(None, kn, vn, pool, bt, np.array([pos + 1], np.int32), P,
                                        W.ROPE_THETA) == oracle.OK
        page, t = bt[0, pos // 16], pos % 16
        changed = np.argwhere(before != pool)
        allowed = set()
        for j in range(8):
            for d in range(64):
                allowed.add((page, j, k_pos(t, d)))
                allowed.add((page, j, v_pos(t, d)))
            for which in ("k", "v"):
                for b in range(4):
                    allowed.add((page, j, scale_pos(t, which) + b))
        assert all(tuple(c) in allowed for c in changed)
        for j in range(8):
            _, vcodes, vsc = read_row(pool, page, j, t, "v")
            want_codes, want_sc = exact_quantise(W.bf16_bits_to_f32(vn[0, j]))
            assert np.array_equal(vcodes.astype(np.int64), want_codes) and float(vsc) == want_sc
            kb = np.array([oracle.f64_to_bf16(y) for y in oracle.rope_head(kn[0, j], pos, W.ROPE_THETA)], np.uint16)
            _, kcodes, ksc = read_row(pool, page, j, t, "k")
            want_codes, want_sc = exact_quantise(W.bf16_bits_to_f32(kb))
            assert np.array_equal(kcodes.astype(np.int64), want_codes) and float(ksc) == want_sc


def random_i8_pool(rng, P):
    """A valid INT8 pool: random codes, positive scales."""
    pool = rng.integers(0, 256, (P, 8, TILE), dtype=np.uint8)
    sc = (np.abs(rng.standard_normal((P, 8, 16, 2))) * 3 / 127 + 1e-3).astype(np.float32)
    pool[:, :, 2048:] = sc.transpose(0, 1, 3, 2).copy().view(np.uint8).reshape(P, 8, 128)  # 16 K, then 16 V scales
    return pool


def dequant_gather(pool, bt_row, L, which):
    out = np.zeros((8, L, 64))
    for t in range(L):
        for j in range(8):
            out[j, t] = read_row(pool, bt_row[t // 16], j, t % 16, which)[0]
    return out


@pytest.mark.parametrize("lens", [[1, 2, 15, 16, 17], [33, 64, 70]])
def test_decode_against_sdpa(lens):
    rng = np.random.default_rng(sum(lens))
    B, MB = len(lens), 5
    P = B * MB
    pool = random_i8_pool(rng, P)
    bt = rng.permutation(P).astype(np.int32).reshape(B, MB)
    q = W.f32_to_bf16_bits(rng.standard_normal((B, 32, 64)).astype(np.float32))
    L = np.array(lens, np.int32)
    out, rc = oracle.decode_gqa_i8(q, pool, bt, L, P, 0.125)
    assert rc == oracle.OK
    for s, n in enumerate(lens):
        k = torch.from_numpy(dequant_gather(pool, bt[s], n, "k"))[None]
        v = torch.from_numpy(dequant_gather(pool, bt[s], n, "v"))[None]
        qq = torch.from_numpy(W.bf16_bits_to_f32(q[s]).astype(np.float64)[:, None, :])[None]
        ref = F.scaled_dot_product_attention(qq, k, v, scale=0.125, enable_gqa=True)[0, :, 0, :].numpy()
        assert np.abs(out[s] - ref).max() < 1e-12


def test_decode_closed_forms():
    rng = np.random.default_rng(21)
    P = 4
    pool = random_i8_pool(rng, P)
    bt = np.array([[2, 0, 1, 3]], np.int32)
    q = W.f32_to_bf16_bits(rng.standard_normal((1, 32, 64)).astype(np.float32))
    # one token: the output is that token's V exactly
    out, rc = oracle.decode_gqa_i8(q, pool, bt, np.array([1], np.int32), P, 0.125)
    assert rc == oracle.OK
    for h in range(32):
        assert np.array_equal(out[0, h], read_row(pool, 2, h // 4, 0, "v")[0])
    # identical V rows (same codes and scale for all 40 tokens): output is that row
    vt = pool[2, :, 1024:2048].copy()
    s0 = pool[2, :, scale_pos(0, "v"):scale_pos(0, "v") + 4].copy()
    for p in range(P):
        pool[p, :, 1024:2048] = vt
        for t in range(16):
            pool[p, :, scale_pos(t, "v"):scale_pos(t, "v") + 4] = s0
    # the V block interleaves the tokens; make every token equal to token 0
    for p in range(P):
        for j in range(8):
            row0 = np.array([pool[p, j, v_pos(0, d)] for d in range(64)], np.uint8)
            for t in range(16):
                for d in range(64):
                    pool[p, j, v_pos(t, d)] = row0[d]
    out, rc = oracle.decode_gqa_i8(q, pool, bt, np.array([40], np.int32), P, 0.125)
    assert rc == oracle.OK
    for h in range(32):
        np.testing.assert_allclose(out[0, h], read_row(pool, 2, h // 4, 0, "v")[0], rtol=1e-14, atol=1e-15)


def test_quantize_pages_places_every_row():
    """The oracle's whole-page quantiser: every (page, head, slot) row of a bf16
    pool pair lands where the header formula says, as the exact-rational
    quantisation of that row; rows holding a NaN keep the bytes they had."""
    rng = np.random.default_rng(31)
    P = 3
    kp = W.f32_to_bf16_bits((rng.standard_normal((P, 8, 16, 64)) * rng.uniform(0.1, 5)).astype(np.float32))
    vp = W.f32_to_bf16_bits(rng.standard_normal((P, 8, 16, 64)).astype(np.float32))
    vp[1, 3, 7, 5] = W.BF16_NAN
    kp[2, 0, 15, :] = 0
    start = rng.integers(0, 256, (P, 8, TILE), dtype=np.uint8)
    pool = oracle.quantize_pages_i8(kp, vp, start.copy())
    for p in range(P):
        for j in range(8):
            for t in range(16):
                for which, src in (("k", kp), ("v", vp)):
                    _, codes, sc = read_row(pool, p, j, t, which)
                    if which == "v" and (p, j, t) == (1, 3, 7):
                        _, codes0, sc0 = read_row(start, p, j, t, which)
                        assert np.array_equal(codes, codes0) and sc.tobytes() == sc0.tobytes()
                        continue
                    want_codes, want_sc = exact_quantise(W.bf16_bits_to_f32(src[p, j, t]))
                    assert np.array_equal(codes.astype(np.int64), want_codes), (p, j, t, which)
                    assert float(sc) == want_sc
