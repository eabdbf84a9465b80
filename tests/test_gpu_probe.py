"""The contiguous-read probe reads every 16-byte vector it is given.  Each of
its threads XORs the words it reads and the sink is written when a thread's
XOR equals the probe's fixed constant.  In an all-zero buffer no thread gets
there; one vector whose four words XOR to the constant, anywhere, makes the
thread that reads it get there.  So the sink is set exactly when that vector
is read, at every position sampled: the edges of the workgroups' chunks, of
their unrolled loops and tails, each unrolled load slot, the last vector and
seeded random ones.  Sizes cover one partial workgroup, whole unrolled groups
plus a tail, and a multi-MiB buffer spread over the full grid."""
import numpy as np
import pytest
import torch

from _gpu_helpers import dev
from _gpu_helpers import guarded_zeros, guarded_flags, to_dev_i32
from paged_kv_gqa_append_amd import binding

pytestmark = pytest.mark.gpu

MAGIC = 0x9E3779B9
THREADS, LOADS, MAX_WG = 256, 8, 2048   # the probe's launch shape


def positions(n_vec):
    """Workgroup w reads vectors [w * per, min(n_vec, (w + 1) * per)): sample the
    edges of the first two and the last chunk, of their unrolled loops and tails,
    each unrolled load slot, and seeded random vectors."""
    unit = THREADS * LOADS
    per = -(-(-(-n_vec // MAX_WG)) // unit) * unit
    grid = -(-n_vec // per)
    assert grid <= MAX_WG and (grid - 1) * per < n_vec
    pos = set()
    for w in {0, 1, grid - 1}:
        lo = w * per
        if lo >= n_vec:
            continue
        hi = min(n_vec, lo + per)
        edge = lo + (hi - lo) // unit * unit
        pos |= {lo, lo + 1, lo + THREADS - 1, hi - 1, edge - 1, edge, edge + 1}
        pos |= {lo + u * THREADS + t for u in range(LOADS) for t in (0, THREADS - 1)}
    pos |= set(np.random.default_rng(n_vec).integers(0, n_vec, size=16).tolist())
    return sorted(p for p in pos if 0 <= p < n_vec)


@pytest.mark.parametrize("n_vec", [1, 37, 256 * 8 * 3 + 5, 256 * 8 * 2048 + 999])
def test_probe_reads_every_vector(n_vec):
    print(f"probe: {n_vec} vectors", flush=True)
    buf = guarded_zeros((n_vec, 4), torch.int32)
    sink = guarded_flags()
    binding.probe_stream_read(buf, sink)
    torch.cuda.synchronize()
    assert int(sink.cpu()[0]) == 0, "sink written for an all-zero buffer"
    words = np.array([0x01234567, 0x89ABCDEF, 0x0F1E2D3C, 0], dtype=np.uint32)
    words[3] = np.uint32(MAGIC) ^ words[0] ^ words[1] ^ words[2]
    magic_vec = to_dev_i32(words.view(np.int32))
    for p in positions(n_vec):
        buf[p] = magic_vec
        sink.zero_()
        binding.probe_stream_read(buf, sink)
        buf[p] = 0
        torch.cuda.synchronize()
        assert int(sink.cpu().numpy().view(np.uint32)[0]) == MAGIC, f"vector {p} of {n_vec} not read"
