"""pa_append_decode_gqa_noalloc against pa_append_decode_gqa (GPU, through the C ABI).

The no-allocation entry point runs the same kernels as the workspace call, with
the library's per-GPU scratch array in place of the caller's workspace, so its
results must be bitwise the workspace call's: the output, the rotated q and
both pools.  Two no-allocation calls run back to back on one stream, the second
on a smaller batch than the first, both with contexts past one partition (so
the scratch really carries partials), in both output dtypes, one of them with a
dispatch order; a batch whose partials would not fit is refused before
anything runs.
"""
import numpy as np
import pytest
import torch

from _gpu_helpers import DeviceCase, guarded_empty, guarded_workspace, rope, to_host_bits
from paged_kv_gqa_append_amd import binding
from paged_kv_gqa_append_amd import workloads as W

pytestmark = pytest.mark.gpu

BIG = [4113, 1, 3000, 2049, 17, 2048, 700, 4096, 33, 2500, 1500, 3999]
SMALL = [2100, 5, 2049]


def _cases():
    big = W.make_decode_case("noalloc_big", 91, BIG, dist="normal", max_blocks=260)
    small = W.make_decode_case("noalloc_small", 92, SMALL, dist="normal", max_blocks=140)
    assert binding.decode_workspace_bytes(big.num_seqs, big.max_blocks) > 0
    assert binding.decode_workspace_bytes(small.num_seqs, small.max_blocks) > 0
    return big, small


def _state(d, out):
    return [to_host_bits(t) if t.dtype == torch.bfloat16 else t.cpu().numpy().view(np.uint32)
            for t in (out, d.q, d.k_pool, d.v_pool)]


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_noalloc_matches_workspace_call(out_dtype):
    table = rope(max_pos=4200)
    big, small = _cases()
    order = binding.dispatch_order_longest_first(big.context_lens) if out_dtype == torch.float32 else None
    print(f"noalloc vs workspace: B={big.num_seqs} then B={small.num_seqs}, out={out_dtype}", flush=True)
    # references: the workspace entry point
    refs = []
    for case, o in ((big, order), (small, None)):
        d = DeviceCase(case)
        out = guarded_empty((case.num_seqs, 32, 64), out_dtype)
        binding.append_decode_gqa(out, d.q, d.k_new, d.v_new, d.k_pool, d.v_pool, d.bt, d.lens, table, case.scale,
                                  workspace=guarded_workspace(case.num_seqs, case.max_blocks), device_flags=d.flags,
                                  dispatch_order=o)
        torch.cuda.synchronize()
        assert int(d.flags.item()) == 0
        refs.append(_state(d, out))
    # the no-allocation calls, back to back on one stream, the second smaller
    runs = []
    for case, o in ((big, order), (small, None)):
        d = DeviceCase(case)
        out = guarded_empty((case.num_seqs, 32, 64), out_dtype)
        binding.append_decode_gqa_noalloc(out, d.q, d.k_new, d.v_new, d.k_pool, d.v_pool, d.bt, d.lens, table,
                                          case.scale, device_flags=d.flags, dispatch_order=o)
        runs.append((d, out))
    torch.cuda.synchronize()
    for (d, out), ref, name in zip(runs, refs, ("first (larger) call", "second (smaller) call")):
        assert int(d.flags.item()) == 0
        for got, want, what in zip(_state(d, out), ref, ("out", "q", "k_pool", "v_pool")):
            assert np.array_equal(got, want), f"{name}: {what} differs from the workspace call"


def test_noalloc_refuses_oversize():
    """Partials beyond the scratch: PA_ERR_WORKSPACE, nothing launched (the pointers are never read)."""
    import ctypes

    lib = binding.lib()
    pp = binding.decode_partition_tokens() // 16
    B, mb = 64, 16 * pp + 1  # 17 partitions of 64 sequences: more than 8 MiB of partials
    assert binding.decode_workspace_bytes(B, mb) > binding.NOALLOC_SCRATCH_BYTES
    F = ctypes.c_void_p(0x7F0000000000)
    rc = lib.pa_append_decode_gqa_noalloc(F, F, F, F, F, F, F, F, F, B, mb, 1 << 16, 16, 4096, 0.125, 0, None, None,
                                          None, None)
    assert rc == binding.PA_ERR_WORKSPACE
