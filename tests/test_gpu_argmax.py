"""GPU parity of pa_argmax against the oracle: the chosen index of every row
is compared bit-exactly (it is integer work; both sides compare the same bf16
or fp32 values, exactly).  Shapes span one and several chunks, a ragged last
chunk, vocabularies that force the scalar path, a misaligned base, and the
full 128,256-entry Llama 3.2 vocabulary; rows carry tied maxima, NaN, -inf,
all-NaN and signed zeros."""
import numpy as np
import pytest
import torch

import oracle
from _gpu_helpers import dev
from _gpu_helpers import guarded_empty, guarded_full, guarded_argmax_workspace, to_dev_bf16, to_dev_f32
from paged_kv_gqa_append_amd import binding
from paged_kv_gqa_append_amd import workloads as W

pytestmark = pytest.mark.gpu

SHAPES = [(1, 1), (7, 7), (6, 16384), (6, 16385), (9, 1001), (64, W.VOCAB_SIZE), (257, 4096)]


def run(x32, dtype, offset=0):
    rows, vocab = x32.shape
    if dtype == torch.bfloat16:
        host = W.f32_to_bf16_bits(x32)
        flat = guarded_empty((rows * vocab + offset,), torch.bfloat16)
        flat[offset:] = torch.from_numpy(host.view(np.int16).ravel()).view(torch.bfloat16).to(dev())
        ref = oracle.argmax(host)
    else:
        flat = guarded_empty((rows * vocab + offset,), torch.float32)
        flat[offset:] = torch.from_numpy(x32.ravel()).to(dev())
        ref = oracle.argmax(x32)
    logits = flat[offset:].view(rows, vocab)
    out = guarded_full((rows,), -7, torch.int32)
    binding.argmax(out, logits, workspace=guarded_argmax_workspace(rows, vocab, dtype))
    torch.cuda.synchronize()
    return out.cpu().numpy(), ref


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_argmax_parity(shape, dtype):
    rows, vocab = shape
    print(f"argmax rows={rows} vocab={vocab} dtype={dtype}", flush=True)
    x = W.argmax_logits(90 + rows + vocab, rows, vocab)
    got, ref = run(x, dtype)
    assert np.array_equal(got, ref), f"{int((got != ref).sum())} rows differ"


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_argmax_misaligned_base_takes_scalar_path(dtype):
    x = W.argmax_logits(91, 6, 16384 + 40)
    got, ref = run(x, dtype, offset=1)
    assert np.array_equal(got, ref)


def test_argmax_bf16_ties_from_rounding():
    """bf16 rounding turns near-equal fp32 maxima into exact ties: the lowest wins."""
    rng = np.random.default_rng(92)
    x = rng.standard_normal((16, 50000)).astype(np.float32)
    for r in range(16):
        pos = np.sort(rng.choice(50000, 5, replace=False))
        x[r, pos] = 9.0 + rng.uniform(0, 0.01, 5).astype(np.float32)   # one bf16 value after rounding
    got, ref = run(x, torch.bfloat16)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_argmax_workspace_reused_and_left_zero(dtype):
    """One workspace, zeroed once, serves calls of shrinking size back to back on
    one stream: every call matches the oracle and the workspace ends all zero
    (the last chunk of each row resets the row's key and arrival count)."""
    rows0, vocab0 = 40, W.VOCAB_SIZE
    ws = guarded_argmax_workspace(rows0, vocab0, dtype)
    assert ws is not None and ws.numel() == 2 * rows0
    for k, (rows, vocab) in enumerate([(40, W.VOCAB_SIZE), (40, W.VOCAB_SIZE), (17, 70001), (3, 16385)]):
        print(f"argmax reuse call {k}: rows={rows} vocab={vocab} dtype={dtype}", flush=True)
        x = W.argmax_logits(93 + k, rows, vocab)
        if dtype == torch.bfloat16:
            host = W.f32_to_bf16_bits(x)
            logits = to_dev_bf16(host)
            ref = oracle.argmax(host)
        else:
            logits = to_dev_f32(x)
            ref = oracle.argmax(x)
        out = guarded_full((rows,), -7, torch.int32)
        binding.argmax(out, logits, workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), ref), f"call {k}"
        assert int(torch.count_nonzero(ws)) == 0, f"workspace not reset after call {k}"
