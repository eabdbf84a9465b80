"""Longest-first dispatch from device memory: pa_order_by_length ranks the
device-resident lengths on the GPU, and every decode entry point takes such an
order (device_order; the binding passes a device tensor given as
dispatch_order).

The order itself is integer work, checked exactly: it is the unique stable
ordering by the header's length classes (longest class first, index order
inside a class), dealt in the header's runs from the long and the short end,
so it equals numpy's stable sort on those classes dealt the same way, for
batches of 1 to 1024 sequences, table widths whose classes hold 1 to 64 pages,
and lengths that are invalid (placed last).  An order moves work in time and
nothing else, so decodes dispatched by it give the bits of slot order: out,
the rotated q and the pools after the append, bf16 and INT8 pages, one and two
partitions per sequence, and the allocation-free fused entry point.  An entry
outside the batch is flagged and never dereferenced."""
import numpy as np
import pytest
import torch

import oracle
from _gpu_helpers import TOL_BF16, assert_close, dev, guarded_empty, guarded_flags, guarded_workspace, rope
from _gpu_helpers import to_dev_bf16, to_dev_i32, to_dev_u8, to_host_bits
from paged_kv_gqa_append_amd import binding
from paged_kv_gqa_append_amd import workloads as W

pytestmark = pytest.mark.gpu


def expected_order(lens, max_blocks, long_run=1, short_run=0):
    """The order the header defines: 64 classes of ceil(max_blocks / 64) pages; class of a valid
    length L: (ceil(L / 16) - 1) // width; invalid lengths class 0; stable, longest class first;
    then dealt long_run from the long end, short_run from the short end, until the ends meet."""
    lens = np.asarray(lens, dtype=np.int64)
    width = -(-max_blocks // 64)
    valid = (lens >= 1) & (lens <= 16 * max_blocks)
    cls = np.where(valid, (-(-lens // 16) - 1) // width, 0)
    ranked = np.lexsort((np.arange(len(lens)), -cls)).astype(np.int32)
    out, a, b = [], 0, len(ranked) - 1
    while a <= b:
        for _ in range(long_run):
            if a <= b:
                out.append(ranked[a])
                a += 1
        for _ in range(short_run):
            if a <= b:
                out.append(ranked[b])
                b -= 1
    return np.array(out, dtype=np.int32), cls


def test_expected_order_runs():
    """The run rule on the header's own example: with runs 3, 2, ten sequences ranked 0..9 are
    dealt 0 1 2 9 8 3 4 5 7 6."""
    lens = 16 * np.arange(10, 0, -1) * 8  # ten distinct classes, longest first
    assert expected_order(lens, 128, 3, 2)[0].tolist() == [0, 1, 2, 9, 8, 3, 4, 5, 7, 6]


@pytest.mark.parametrize("n", [1, 2, 63, 64, 65, 256, 1000, 1024])
@pytest.mark.parametrize("max_blocks", [1, 8, 64, 65, 128, 129, 4096])
@pytest.mark.parametrize("runs", [(1, 0), (3, 2), (1, 1), (4, 1), (64, 64)])
def test_order_by_length_exact(n, max_blocks, runs):
    rng = np.random.default_rng(n * 7919 + max_blocks)
    top = 16 * max_blocks
    lens = rng.integers(1, top + 1, size=n)
    k = rng.random(n)
    lens = np.where(k < 0.1, rng.choice([0, -7, top + 1, 2**31 - 1, -2**31], size=n), lens)  # invalid ones
    lens = np.where((k >= 0.1) & (k < 0.2), rng.choice([1, 16, 17, top], size=n), lens)  # edges
    lens = lens.astype(np.int32)
    want, cls = expected_order(lens, max_blocks, *runs)
    order = guarded_empty((n,), torch.int32)
    binding.order_by_length(to_dev_i32(lens), max_blocks, order, *runs)
    got = order.cpu().numpy()
    assert np.array_equal(np.sort(got), np.arange(n)), "not a permutation"
    if runs[1] == 0:
        assert np.all(np.diff(cls[got]) <= 0), "classes not descending"
    assert np.array_equal(got, want)


def test_order_by_length_empty_and_lengths_untouched():
    lens = to_dev_i32(np.array([5, 700, 33], np.int32))
    binding.order_by_length(lens, 128)
    assert lens.cpu().numpy().tolist() == [5, 700, 33]
    binding.order_by_length(torch.empty(0, dtype=torch.int32, device=dev()), 128)
    torch.cuda.synchronize()


def lengths(n, seed, top):
    rng = np.random.default_rng(seed)
    lens = np.clip(np.rint(np.exp(rng.normal(6.0, 1.0, size=n))), 1, 2048).astype(np.int32)
    edges = [1, 2, 16, 17, 32, 33, 2047, 2048, top]
    lens[rng.choice(n, size=min(n, len(edges)), replace=False)] = edges[:min(n, len(edges))]
    return lens


def run(case, kv, fused, order, pool_i8, table, lens=None, noalloc=False):
    lens = case.context_lens if lens is None else lens
    pools = [to_dev_u8(pool_i8)] if kv == "int8" else [to_dev_bf16(case.k_pool), to_dev_bf16(case.v_pool)]
    q = to_dev_bf16(case.q[0])
    dbt, dlens = to_dev_i32(case.block_tables[0]), to_dev_i32(lens)
    kn, vn = to_dev_bf16(case.k_new[0]), to_dev_bf16(case.v_new[0])
    out = guarded_empty((case.num_seqs, 32, 64), torch.bfloat16)
    ws = guarded_workspace(case.num_seqs, case.max_blocks)
    flags = guarded_flags()
    if isinstance(order, str):  # computed on the device from the lengths the decode reads
        runs = (3, 2) if order == "device32" else (1, 0)
        order = binding.order_by_length(dlens, case.max_blocks, guarded_empty((case.num_seqs,), torch.int32), *runs)
    kw = dict(dispatch_order=order, device_flags=flags)
    if noalloc:
        binding.append_decode_gqa_noalloc(out, q, kn, vn, pools[0], pools[1], dbt, dlens, table, case.scale, **kw)
    elif kv == "int8":
        if fused:
            binding.append_decode_gqa_i8(out, q, kn, vn, pools[0], dbt, dlens, table, case.scale, workspace=ws,
                                         **kw)
        else:
            binding.decode_gqa_i8(out, q, pools[0], dbt, dlens, case.scale, workspace=ws, **kw)
    elif fused:
        binding.append_decode_gqa(out, q, kn, vn, pools[0], pools[1], dbt, dlens, table, case.scale, workspace=ws,
                                  **kw)
    else:
        binding.decode_gqa(out, q, pools[0], pools[1], dbt, dlens, case.scale, workspace=ws, **kw)
    torch.cuda.synchronize()
    return (to_host_bits(out), to_host_bits(q), [p.view(torch.uint8).cpu().numpy() for p in pools],
            int(flags.item()))


def assert_same(a, b, what):
    assert a[3] == b[3], f"{what}: device flags differ ({a[3]:#x} against {b[3]:#x})"
    assert np.array_equal(a[0], b[0]), f"{what}: out differs"
    assert np.array_equal(a[1], b[1]), f"{what}: rotated q differs"
    for x, y in zip(a[2], b[2]):
        assert np.array_equal(x, y), f"{what}: pool differs"


CASES = {  # name: (sequences, max_blocks): one partition per sequence, then two
    "n65": (65, 128),
    "n256": (256, 128),
    "n40_two_parts": (40, 256),
}


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("kv", ["bf16", "int8"])
@pytest.mark.parametrize("fused", [False, True])
def test_device_order_equals_slot_order(name, kv, fused):
    n, mb = CASES[name]
    print(f"device order: case={name} kv={kv} fused={fused}", flush=True)
    case = W.make_decode_case(f"devorder_{name}", 600 + n, lengths(n, 700 + n, 16 * mb), dist="normal",
                              max_blocks=mb)
    pool_i8 = oracle.quantize_pages_i8(case.k_pool, case.v_pool) if kv == "int8" else None
    table = rope(16 * mb + 64)
    base = run(case, kv, fused, None, pool_i8, table)
    assert base[3] == 0
    perm = np.random.default_rng(n).permutation(n).astype(np.int32)
    for what, order in (("order_by_length", "device"), ("runs 3, 2", "device32"), ("random", to_dev_i32(perm))):
        assert_same(base, run(case, kv, fused, order, pool_i8, table), f"{name} {kv} fused={fused} {what}")
    if not fused:
        if kv == "int8":
            ref, rc = oracle.decode_gqa_i8(case.q[0], pool_i8, case.block_tables[0], case.context_lens,
                                           case.num_pages, case.scale)
        else:
            ref, rc = oracle.decode_gqa(case.q[0], case.k_pool, case.v_pool, case.block_tables[0],
                                        case.context_lens, case.num_pages, case.scale)
        assert rc == oracle.OK
        assert_close(W.bf16_bits_to_f32(base[0]).astype(np.float64), ref, TOL_BF16, f"{name} {kv}")


def test_device_order_noalloc():
    n, mb = 100, 256
    case = W.make_decode_case("devorder_noalloc", 811, lengths(n, 812, 16 * mb), dist="normal", max_blocks=mb)
    table = rope(16 * mb + 64)
    base = run(case, "bf16", True, None, None, table, noalloc=True)
    assert base[3] == 0
    assert_same(base, run(case, "bf16", True, "device", None, table, noalloc=True), "noalloc")


@pytest.mark.parametrize("kv", ["bf16", "int8"])
def test_device_order_bad_entries_flagged(kv):
    """Entries outside [0, n) (negative, n, large) are never used as sequence indices: their
    workgroups only raise PA_DEVERR_DISPATCH_ORDER (the canaries around every buffer stay
    intact, checked after the test)."""
    n, mb = 70, 256
    case = W.make_decode_case("devorder_bad", 913, lengths(n, 914, 16 * mb), dist="normal", max_blocks=mb)
    pool_i8 = oracle.quantize_pages_i8(case.k_pool, case.v_pool) if kv == "int8" else None
    table = rope(16 * mb + 64)
    bad = np.arange(n, dtype=np.int32)
    bad[[3, 40, 69]] = [-1, n, 1 << 30]
    for fused in (False, True):
        got = run(case, kv, fused, to_dev_i32(bad), pool_i8, table)
        assert got[3] == binding.PA_DEVERR_DISPATCH_ORDER, f"fused={fused}: flags {got[3]:#x}"
