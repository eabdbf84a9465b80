"""Helpers shared by the GPU parity tests (device upload, bf16 ulp distance, tolerances)."""
import numpy as np
import torch

from paged_kv_gqa_append_amd import workloads as W

# Tolerances of the method's outputs against the fp64 oracle, elementwise:
# |gpu - ref| <= atol + rtol * |ref|.
TOL_BF16 = (1e-2, 1e-2)
TOL_FP32 = (2e-3, 2e-3)


def dev():
    return torch.device("cuda", 0)


def to_dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev())


def to_dev_i32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev())


def to_host_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def to_host_f64(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return W.bf16_bits_to_f32(to_host_bits(t)).astype(np.float64)
    return t.detach().cpu().numpy().astype(np.float64)


def bf16_ulp_distance(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    def ordered(x):
        u = x.astype(np.int32)
        mag = u & 0x7FFF
        return np.where(u & 0x8000, -mag, mag)

    return np.abs(ordered(a) - ordered(b))


def bf16_ulp(bits: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values at each (finite) value."""
    v = np.abs(W.bf16_bits_to_f32(bits).astype(np.float64))
    _, e = np.frexp(np.where(v > 0, v, 1.0))
    return np.ldexp(1.0, np.maximum(e - 1, -126) - 7)


def assert_rope_close(gpu_bits: np.ndarray, ref_bits: np.ndarray, max_abs_input: float, what=""):
    """Rotated bf16 rows: the device rotates in fp32 with a rounded (cos, sin)
    table, the oracle in fp64; each result is rounded once to bf16.  They may
    differ by one bf16 step plus the fp32 evaluation error of x_i cos - x_j sin,
    at most ~2^-22 (|x_i| + |x_j|) <= 2^-21 max|x|, which spans several steps
    only when the two terms cancel to a tiny result."""
    g = W.bf16_bits_to_f32(gpu_bits).astype(np.float64)
    r = W.bf16_bits_to_f32(ref_bits).astype(np.float64)
    bound = bf16_ulp(ref_bits) + 2.0 ** -21 * max_abs_input
    bad = np.abs(g - r) > bound
    assert not bad.any(), f"{what}: {int(bad.sum())} rotated elements outside 1 ulp + fp32 bound"


def assert_close(got: np.ndarray, ref: np.ndarray, tol, what=""):
    atol, rtol = tol
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    bound = atol + rtol * np.abs(ref)
    bad = err > bound
    if bad.any():
        i = np.argmax(err - bound)
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; worst idx "
                             f"{np.unravel_index(i, err.shape)} got {got.flat[i]} ref {ref.flat[i]}")
    return float(err.max()) if err.size else 0.0


def rope(max_pos=W.MAX_CONTEXT + 64):
    from paged_kv_gqa_append_amd import binding

    return binding.rope_table(max_pos, W.ROPE_THETA, dev())


class DeviceCase:
    """Device copy of one layer of a host PagedCase."""

    def __init__(self, case: W.PagedCase, layer: int = 0):
        self.case = case
        self.layer = layer
        self.k_pool = to_dev_bf16(case.k_pool)
        self.v_pool = to_dev_bf16(case.v_pool)
        self.q = to_dev_bf16(case.q[layer])
        self.k_new = to_dev_bf16(case.k_new[layer])
        self.v_new = to_dev_bf16(case.v_new[layer])
        self.bt = to_dev_i32(case.block_tables[layer])
        self.lens = to_dev_i32(case.context_lens)
        self.flags = torch.zeros(1, dtype=torch.int32, device=dev())
