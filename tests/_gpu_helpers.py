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


# ---- guard bands -------------------------------------------------------------
# Every device buffer the GPU tests hand to the library (inputs, outputs, pools,
# tables, flags) is the middle of a larger allocation whose first and last
# GUARD_BYTES hold a fixed canary: bytes A5 7F repeated, which read as NaN in
# bf16 (0x7FA5) and fp32 (0x7FA57FA5).  A kernel store that runs past an output
# row, a (page, head) tile or a chunk lands in a canary, and so does a read-
# modify-write of a neighbouring buffer; check_guards(), run after every GPU
# test (tests/conftest.py), finds it.  The canaries are never legitimately
# written, so one check at the end of a test covers every call it made,
# aliased and device-error calls included.
GUARD_BYTES = 4096
_GUARD_PATTERN = np.tile(np.array([0xA5, 0x7F], np.uint8), GUARD_BYTES // 2)
_guarded = []


def guarded_empty(shape, dtype) -> torch.Tensor:
    """Uninitialised device tensor of shape/dtype between two canary regions (16-byte aligned)."""
    shape = tuple(int(x) for x in shape)
    el = torch.empty((), dtype=dtype).element_size()
    nbytes = int(np.prod(shape, dtype=np.int64)) * el
    tail = GUARD_BYTES + (-nbytes) % 16
    buf = torch.empty(GUARD_BYTES + nbytes + tail, dtype=torch.uint8, device=dev())
    pat = torch.from_numpy(np.resize(_GUARD_PATTERN, tail)).to(dev())
    buf[:GUARD_BYTES] = pat[:GUARD_BYTES]
    buf[GUARD_BYTES + nbytes:] = pat
    _guarded.append((buf, nbytes, tail))
    return buf[GUARD_BYTES:GUARD_BYTES + nbytes].view(dtype).view(shape)


def guarded_full(shape, value, dtype) -> torch.Tensor:
    return guarded_empty(shape, dtype).fill_(value)


def guarded_zeros(shape, dtype) -> torch.Tensor:
    return guarded_full(shape, 0, dtype)


def guarded_clone(t: torch.Tensor) -> torch.Tensor:
    return guarded_empty(t.shape, t.dtype).copy_(t)


def guarded_flags() -> torch.Tensor:
    """A device_flags word (int32, zero)."""
    return guarded_zeros((1,), torch.int32)


def check_guards() -> int:
    """Assert every canary written since the last check is intact; forget the buffers.
    Returns how many buffers were checked."""
    n = len(_guarded)
    if not n:
        return 0
    torch.cuda.synchronize()
    bad = []
    for buf, nbytes, tail in _guarded:
        head = buf[:GUARD_BYTES].cpu().numpy()
        back = buf[GUARD_BYTES + nbytes:].cpu().numpy()
        if not np.array_equal(head, _GUARD_PATTERN):
            bad.append(f"{nbytes}-byte buffer: {int((head != _GUARD_PATTERN).sum())} canary bytes changed before it")
        if not np.array_equal(back, np.resize(_GUARD_PATTERN, tail)):
            bad.append(f"{nbytes}-byte buffer: {int((back != np.resize(_GUARD_PATTERN, tail)).sum())} canary bytes "
                       "changed after it")
    _guarded.clear()
    assert not bad, "guard band overwritten: " + "; ".join(bad)
    return n


def to_dev_bf16(bits: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(bits).view(np.int16)
    return guarded_empty(a.shape, torch.bfloat16).copy_(torch.from_numpy(a).view(torch.bfloat16))


def to_dev_i32(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a, dtype=np.int32)
    return guarded_empty(a.shape, torch.int32).copy_(torch.from_numpy(a))


def to_dev_u8(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a, dtype=np.uint8)
    return guarded_empty(a.shape, torch.uint8).copy_(torch.from_numpy(a))


def to_dev_f32(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a, dtype=np.float32)
    return guarded_empty(a.shape, torch.float32).copy_(torch.from_numpy(a))


def guarded_workspace(num_seqs: int, max_blocks: int):
    """The decode workspace (pa_decode_workspace_bytes), between canaries; None when none is needed."""
    from paged_kv_gqa_append_amd import binding

    n = binding.decode_workspace_bytes(num_seqs, max_blocks)
    return None if n == 0 else guarded_empty((n // 4,), torch.float32)


def guarded_argmax_workspace(rows: int, vocab: int, dtype):
    """The argmax workspace (zeroed once, as its contract asks), between canaries; None when none is needed."""
    from paged_kv_gqa_append_amd import binding

    code = binding.PA_LOGITS_BF16 if dtype == torch.bfloat16 else binding.PA_LOGITS_FP32
    n = int(binding.lib().pa_argmax_workspace_bytes(int(rows), int(vocab), code))
    return None if n == 0 else guarded_zeros((n // 8,), torch.int64)


def guarded_pool(spec, which: str) -> torch.Tensor:
    """A full-size seeded pool (workloads.fill_pool_device) drawn into a guarded buffer."""
    pool = guarded_empty((spec.num_pages, W.NUM_KV_HEADS, W.PAGE_SIZE, W.HEAD_DIM), torch.bfloat16)
    return W.fill_pool_device(spec, dev(), which, out=pool)


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


def assert_rope_equal(gpu_bits: np.ndarray, ref_bits: np.ndarray, what=""):
    """Rotated bf16 rows (and every other byte of the arrays) bit for bit: the
    device evaluates the rotation with the fp64 operations of the oracle's
    definition (each product and the sum rounded on its own, then one rounding
    to bf16) from a table of the same libm values, so nothing may differ."""
    assert gpu_bits.shape == ref_bits.shape, (gpu_bits.shape, ref_bits.shape)
    bad = gpu_bits != ref_bits
    if bad.any():
        i = np.argmax(bad)
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} elements differ; first at "
                             f"{np.unravel_index(i, bad.shape)}: gpu {int(gpu_bits.flat[i]):#06x} "
                             f"ref {int(ref_bits.flat[i]):#06x}")


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

    return guarded_clone(binding.rope_table(max_pos, W.ROPE_THETA, dev()))


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
        self.flags = guarded_flags()
