"""Pins for the oracle's argmax over logit rows.

The pages' CPU argmax (tiny-vllm ch.2, section "Preallocating the 16 compute
buffers") scans the row with a strict greater-than from element 0, so the
first maximum wins; samir-vllm (section "Architecture et flux d'inference")
runs it on the GPU.  Reading for NaN (the pages are silent): NaN entries are
never chosen, an all-NaN row gives 0.

* numpy's argmax (first occurrence of the maximum) on NaN-free rows, bf16 and
  fp32, at the full 128,256-entry vocabulary;
* the pages' own scan (start at element 0, strict >) on NaN-free rows;
* constructed ties, signed zeros, -inf and NaN placements with hand-known answers.
"""
import numpy as np
import pytest

import oracle
from paged_kv_gqa_append_amd import workloads as W

VOCAB = 128256


def pages_scan(row):
    best, idx = float(row[0]), 0
    for i in range(1, len(row)):
        if float(row[i]) > best:
            best, idx = float(row[i]), i
    return idx


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_matches_numpy_first_maximum(dtype):
    rng = np.random.default_rng(3)
    x = rng.standard_normal((6, VOCAB)).astype(np.float32)
    x[2, 1000] = x[2, 77] = 9.0          # an exact tie at two places: 77 wins
    if dtype == "bf16":
        bits = W.f32_to_bf16_bits(x)      # bf16 rounding creates many more ties
        vals = W.bf16_bits_to_f32(bits)
        got = oracle.argmax(bits)
    else:
        vals = x
        got = oracle.argmax(x)
    assert np.array_equal(got, np.argmax(vals, axis=1))
    assert got[2] == 77


def test_matches_the_pages_scan():
    rng = np.random.default_rng(4)
    for n in (1, 2, 3, 17, 1000):
        x = W.f32_to_bf16_bits(rng.integers(-3, 4, size=(5, n)).astype(np.float32))  # many ties
        got = oracle.argmax(x)
        vals = W.bf16_bits_to_f32(x)
        for r in range(5):
            assert got[r] == pages_scan(vals[r])


def test_hand_cases():
    nan, inf = np.float32("nan"), np.float32("inf")
    rows = [
        ([-0.0, 0.0, -1.0], 0),           # -0 == +0: the first wins
        ([0.0, -0.0, -1.0], 0),
        ([-inf, -inf, -inf], 0),          # all equal
        ([nan, -inf, -inf], 1),           # NaN is never chosen
        ([nan, nan, nan], 0),             # nothing but NaN: 0
        ([1.0, nan, 2.0, nan, 2.0], 2),
        ([3.0, inf, inf, 5.0, nan], 1),
        ([-5.0, -4.0, -4.0, -7.0, -4.5], 1),
    ]
    for vals, want in rows:
        x = np.array([vals], np.float32)
        assert oracle.argmax(x)[0] == want, vals
        assert oracle.argmax(W.f32_to_bf16_bits(x))[0] == want, vals


def test_single_column_and_shapes():
    x = np.array([[5.0], [-1.0]], np.float32)
    assert list(oracle.argmax(x)) == [0, 0]
    with pytest.raises(ValueError):
        oracle.argmax(np.zeros((2, 0), np.float32))
