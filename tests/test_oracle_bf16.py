"""Pins for the oracle's bf16 storage rounding (one-step fp64 -> bf16, ties to even).

The rotated K and q rows are stored as bf16 (tiny-vllm ch.2, opening section:
every activation is bfloat16, 1 sign, 8 exponent, 7 mantissa bits).  These
tests tie the oracle's rounding to torch's float32 -> bfloat16 conversion on
every float32 input and to hand-built halfway cases for fp64 inputs.
"""
import math
import struct

import numpy as np
import pytest
import torch


def f32_bits(x: float) -> int:
    return struct.unpack("<I", struct.pack("<f", x))[0]


def test_bf16_to_f64_all_patterns(oracle_lib):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle_lib.bf16_to_f64(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_round_matches_torch_on_float32_inputs(oracle_lib):
    rng = np.random.default_rng(123)
    # magnitudes over the whole float32 range, plus random mantissas (many near ties)
    exps = rng.integers(-149, 128, size=20000)
    mant = rng.random(20000) + 1.0
    x = (mant * np.exp2(exps.astype(np.float64))).astype(np.float32)
    x = x * np.where(rng.random(20000) < 0.5, -1.0, 1.0).astype(np.float32)
    # exact ties: bf16 value + half a bf16 step (representable in float32)
    base = rng.integers(0x0080, 0x7F00, size=3000).astype(np.uint32) << 16
    ties = (base | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, np.array([0.0, -0.0, 1e-45, -1e-45, 3.4e38, -3.4e38], np.float32)])
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle_lib.f64_to_bf16(float(v)) for v in x], dtype=np.uint16)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, f"{bad.size} mismatches, e.g. x={x[bad[:3]]} got={got[bad[:3]]} ref={ref[bad[:3]]}"


@pytest.mark.parametrize("k", [0, 1, 2, 37, 126])
def test_halfway_cases_fp64(oracle_lib, k):
    # values 1.m * 2^e: the bf16 step at [1, 2) is 2^-7
    step = 2.0 ** -7
    lo = 1.0 + k * step
    hi = lo + step
    mid = lo + step / 2
    even = lo if (k % 2 == 0) else hi
    assert oracle_lib.f64_to_bf16(mid) == f32_bits(even) >> 16
    assert oracle_lib.f64_to_bf16(mid + 2.0 ** -40) == f32_bits(hi) >> 16
    assert oracle_lib.f64_to_bf16(mid - 2.0 ** -40) == f32_bits(lo) >> 16
    assert oracle_lib.f64_to_bf16(-mid) == (f32_bits(-even) >> 16)


def test_no_double_rounding(oracle_lib):
    # 1 + 2^-8 + 2^-30: above the bf16 tie, but rounds to the tie in float32.
    x = 1.0 + 2.0 ** -8 + 2.0 ** -30
    assert oracle_lib.f64_to_bf16(x) == f32_bits(1.0 + 2.0 ** -7) >> 16
    via_f32 = torch.tensor([x], dtype=torch.float32).to(torch.bfloat16).view(torch.int16).item() & 0xFFFF
    assert via_f32 == f32_bits(1.0) >> 16  # documents why one-step rounding matters


def test_specials(oracle_lib):
    assert oracle_lib.f64_to_bf16(math.inf) == 0x7F80
    assert oracle_lib.f64_to_bf16(-math.inf) == 0xFF80
    assert oracle_lib.f64_to_bf16(math.nan) & 0x7FC0 == 0x7FC0
    assert oracle_lib.f64_to_bf16(-0.0) == 0x8000
    big = (2.0 - 2.0 ** -7) * 2.0 ** 127  # largest finite bf16
    assert oracle_lib.f64_to_bf16(big) == 0x7F7F
    assert oracle_lib.f64_to_bf16(big + 2.0 ** 119) == 0x7F80  # exactly half a step above: tie -> even (inf)
    assert oracle_lib.f64_to_bf16(1e300) == 0x7F80
    # smallest bf16 subnormal is 2^-133; half of it ties to zero, a hair more rounds up
    assert oracle_lib.f64_to_bf16(2.0 ** -133) == 0x0001
    assert oracle_lib.f64_to_bf16(2.0 ** -134) == 0x0000
    assert oracle_lib.f64_to_bf16(2.0 ** -134 * (1 + 2.0 ** -20)) == 0x0001
