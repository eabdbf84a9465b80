#!/usr/bin/env python3
"""Benchmark: paged GQA decode with KV append on one MI355X.

Headline workload (one "step"): 64 sequences at context 2048 (2047 cached
tokens + the one appended this step), 16 layers, 32 q / 8 KV heads, head dim
64, bf16 K/V ~N(0,1) in a pool of 64 x 128 x 16 = 131072 pages whose ids are a
random permutation.  A step runs, for every layer, the append of the new token
(RoPE-rotated K and V written into its page, q rotated in place) and the paged
decode attention: by default as one pa_append_decode_gqa launch per layer;
the same step made of the two separate calls (pa_append_kv_rope, then
pa_decode_gqa) is timed too and reported beside it.  Inputs are resident in
HBM before timing starts.

Prints ONE JSON line.  value = algorithmic KV bytes read per step (tokens
attended x 2048 B x layers) / step time, in GB/s; tokens/s = sequences /
step time.  The roofline object reports the decode kernel alone: its
algorithmic bytes per launch over its mean duration, from the HIP events that
bracket the timed steps on the stream it runs on (the fused step is nothing
but that kernel, once per layer).  Warmup runs until the GPU's clocks have
settled (100 ms of work unless --warmup is given).  roofline.stream_read is the
read ceiling at the same size: pa_probe_stream_read reads the same bytes per
launch as one contiguous stream, one launch per layer over different chunks of
the same pools, timed the same way.  cpu_baseline times the fp64 CPU oracle
(append + decode) on a bounded sample of the same workload.

Without --config the line also carries, under "secondary", one object per
other workload: batch-64 with INT8 pages; the ragged batch-256 in bf16 and
INT8 (slot order, and longest first with the sort inside the timed step);
batch-8 and tiny, warm and cold; the chunked prefill; the greedy argmax, warm
and cold.  Every object (the headline too) carries its time, throughput,
roofline fraction, a bounded cpu_baseline and an "accuracy" object: the
outputs of one more call, made after the timed steps, against the fp64
oracle run on the same inputs (max_abs_err, max_rel_err, and the largest
error over the tolerance atol + rtol |ref|, which must stay <= 1).
--config NAME prints that workload alone, in the headline's form.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBPS = 8000.0
# decode workgroups resident at once: 2 per CU (8 waves each, at most 4 waves per SIMD), 256 CUs
RESIDENT_DECODE_WGS = 512
# (long_run, short_run) of the ragged steps' device order, per page format: ragged batches of 256
# sequences over four seeds, us per launch against plain longest first (1, 0): bf16 (3, 2) 2.3-2.6 %
# faster, (2, 1) 1.2-2.0 %, (1, 1) 7 % slower; INT8 (4, 1) 0-1 % faster, (3, 2) and (3, 1) slower.
ORDER_RUNS = {"bf16": (3, 2), "int8": (4, 1)}
# sources each fused decode kernel is compiled from (its traffic figure is tied to them),
# and the committed rocprofv3 summary that holds that figure
TRAFFIC = {
    "bf16": (("pa_decode.hip", "pa_decode_core.h", "pa_device.h"), "decode_batch64_pmc_traffic.md"),
    "int8": (("pa_i8.hip", "pa_decode_core.h", "pa_device.h"), "decode_batch64_i8_pmc_traffic.md"),
    "argmax": (("pa_argmax.hip", "pa_device.h"), "argmax_batch64_pmc_traffic.md"),
}
# K+V bytes per (token, layer): 8 heads x 2 x 64 x 2 B in bf16; 8 tiles' share (2176 B / 16 slots) in INT8
KV_TOKEN_BYTES = {"bf16": 2048, "int8": 8 * 2176 // 16}
METRIC = "paged GQA decode: KV-read GB/s and % of HBM peak; decode tokens/s (1 GPU)"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warmup steps; by default, steps until 100 ms of work have run (at least 5), "
                         "since the GPU's clocks take about 10-20 ms of sustained load to settle")
    ap.add_argument("--config", default=None,
                    choices=["batch64", "batch256", "batch8", "tiny", "prefill", "argmax"],
                    help="one workload alone: decode workloads, 'prefill': 4 x (1536 cached + 512-token chunk) "
                         "chunked prefill, or 'argmax': greedy choice over 64 x 128,256 bf16 logits; by default "
                         "the batch-64 bf16 headline plus every other workload as secondary objects")
    ap.add_argument("--path", default="fused", choices=["fused", "separate"])
    ap.add_argument("--kv", default="bf16", choices=["bf16", "int8"],
                    help="K/V page format: bf16 pools, or INT8 tiles (codes + one fp32 scale per token and head), "
                         "quantised on the device from the same bf16 pages before timing")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (3 times): under rocprofv3 --pmc its FETCH_SIZE / "
                         "WRITE_SIZE give the factor that scales those counters to bytes")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU work of the oracle sample")
    ap.add_argument("--cpu-seconds-secondary", type=float, default=3.0,
                    help="target CPU work of each secondary workload's oracle sample")
    ap.add_argument("--no-accuracy", action="store_true", help="skip the oracle comparisons")
    return ap.parse_args()


def build_workload(name, device):
    import torch

    from paged_kv_gqa_append_amd import workloads as W

    if name == "batch64":
        spec = W.batch64_spec()
    elif name == "batch256":
        spec = W.batch256_spec()
    elif name == "batch8":
        c = W.batch8_decode(poison=False)
        spec = W.DeviceCaseSpec("batch8_decode", 1, c.num_seqs, c.max_blocks, c.num_pages, c.context_lens,
                                c.block_tables, c.seed)
    else:
        c = W.tiny_decode(poison=False)
        spec = W.DeviceCaseSpec("tiny_decode", 1, c.num_seqs, c.max_blocks, c.num_pages, c.context_lens,
                                c.block_tables, c.seed)
    k_pool = W.fill_pool_device(spec, device, "k")
    v_pool = W.fill_pool_device(spec, device, "v")
    rows = [spec.host_rows(l) for l in range(spec.num_layers)]

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)

    layers = []
    for l in range(spec.num_layers):
        q, kn, vn = rows[l]
        layers.append(dict(q=up(q), k_new=up(kn), v_new=up(vn),
                           bt=torch.from_numpy(spec.block_tables[l]).to(device),
                           out=torch.empty((spec.num_seqs, 32, 64), dtype=torch.bfloat16, device=device)))
    lens = torch.from_numpy(spec.context_lens).to(device)
    return spec, k_pool, v_pool, layers, lens, rows


def warm_up(fn, torch, n):
    """Run fn untimed n times, or (n None) in rounds of 5 until 100 ms have passed; the count run."""
    if n is not None:
        for _ in range(n):
            fn()
        torch.cuda.synchronize()
        return n
    t0, k = time.perf_counter(), 0
    while True:
        for _ in range(5):
            fn()
        k += 5
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= 0.1:
            return k


def host_cpu_model():
    """The host CPU's model name, as /proc/cpuinfo gives it (None if unreadable)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def measured_traffic(kv="bf16", profiles_dir=None):
    """HBM bytes per fused decode launch from the committed rocprofv3 PMC summary.

    The summary records the sha256 of the decode kernel's sources (the files
    of TRAFFIC[kv], concatenated in that order) it was taken with; if they
    have changed since, the figure no longer applies and None is returned.
    """
    import hashlib
    import re

    here = os.path.dirname(os.path.abspath(__file__))
    csrc = os.path.join(here, "paged_kv_gqa_append_amd", "csrc")
    sources, summary = TRAFFIC[kv]
    summ = os.path.join(profiles_dir or os.path.join(here, "profiles"), summary)
    try:
        text = open(summ).read()
        h = hashlib.sha256()
        for name in sources:
            h.update(open(os.path.join(csrc, name), "rb").read())
        digest = h.hexdigest()
    except OSError:
        return None
    m_src = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    m_val = re.search(r"traffic_bytes_per_launch:\s*(\d+)", text)
    if not m_src or not m_val or m_src.group(1) != digest:
        return None
    return int(m_val.group(1))


def stream_read_ceiling(buffers, chunk_bytes, per_step, steps, torch, binding, device, stream):
    """Read bandwidth of the plain contiguous-read probe (pa_probe_stream_read) over chunks of
    chunk_bytes, per_step launches back to back per step, each on a different chunk of the given
    device buffers (as a decode step reads different pages in every layer, so no launch finds the
    previous one's bytes in cache).  Returns (GB/s, mean us per launch, distinct chunks); with
    fewer distinct chunks than launches per step (small pools) the chunks repeat and may be read
    from the 256 MB MALL, as the decode's own pages are then."""
    chunk = chunk_bytes // 16 * 16
    flat = [b.view(torch.uint8).reshape(-1) for b in buffers]
    chunks = [f[o:o + chunk] for f in flat for o in range(0, f.numel() - chunk + 1, chunk)]
    if not chunks or chunk == 0:
        return None, None, 0
    sink = torch.zeros(1, dtype=torch.int32, device=device)
    seq = [chunks[i % len(chunks)] for i in range(per_step)]

    def step():
        for c in seq:
            binding.probe_stream_read(c, sink, stream=stream)

    warm_up(step, torch, None)
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(steps):
        step()
    b.record(stream)
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / (steps * per_step)
    return chunk / (us * 1e-6) / 1e9, us, min(len(chunks), per_step)


def host_case(spec, k_pool, v_pool, rows, layer, seqs):
    """Host copies of what the oracle needs for the given sequences of one layer: the pages they
    use (renumbered densely), their block tables, q / k_new / v_new rows and lengths."""
    import torch

    bt = spec.block_tables[layer][seqs]
    used = np.unique(bt[bt >= 0])
    remap = np.full(spec.num_pages, -1, np.int64)
    remap[used] = np.arange(len(used))
    idx = torch.from_numpy(used).to(k_pool.device)
    kp = k_pool.index_select(0, idx).cpu().view(torch.int16).numpy().view(np.uint16).copy()
    vp = v_pool.index_select(0, idx).cpu().view(torch.int16).numpy().view(np.uint16).copy()
    bt2 = np.where(bt >= 0, remap[np.maximum(bt, 0)], -1).astype(np.int32)
    q, kn, vn = rows[layer]
    return kp, vp, bt2, q[seqs].copy(), kn[seqs].copy(), vn[seqs].copy(), spec.context_lens[seqs].copy(), len(used)


def cpu_baseline(spec, k_pool, v_pool, rows, target_s, kv="bf16"):
    """Time the fp64 oracle's append + decode on whole layers of the workload (host cores).

    For INT8 pages the oracle quantises the layer's bf16 pages itself (untimed)
    and its INT8 append + decode are timed."""
    import oracle

    # sample: whole layers of the workload, in order, until the CPU budget is spent
    def run(seqs, layer):
        kp, vp, bt, q, kn, vn, lens, npg = host_case(spec, k_pool, v_pool, rows, layer, seqs)
        if kv == "int8":
            pool = oracle.quantize_pages_i8(kp, vp)
            t0 = time.perf_counter()
            rc = oracle.append_kv_rope_i8(q, kn, vn, pool, bt, lens, npg, spec.theta)
            out, rc2 = oracle.decode_gqa_i8(q, pool, bt, lens, npg, spec.scale)
        else:
            t0 = time.perf_counter()
            rc = oracle.append_kv_rope(q, kn, vn, kp, vp, bt, lens, npg, spec.theta)
            out, rc2 = oracle.decode_gqa(q, kp, vp, bt, lens, npg, spec.scale)
        dt = time.perf_counter() - t0
        assert rc == oracle.OK and rc2 == oracle.OK
        return dt, int(lens.astype(np.int64).sum())

    B = spec.num_seqs
    seqs = np.arange(B)
    total_dt, total_tokens, layers_done = 0.0, 0, 0
    for layer in range(spec.num_layers):
        dt, tokens = run(seqs, layer)
        total_dt += dt
        total_tokens += tokens
        layers_done += 1
        if total_dt >= target_s:
            break
    kv_bytes = total_tokens * KV_TOKEN_BYTES[kv]
    return {"value": round(kv_bytes / total_dt / 1e9, 4), "unit": "GB/s", "cores": oracle.num_threads(),
            "cpu_model": host_cpu_model(), "kind": "oracle", "seconds": round(total_dt, 3),
            "tokens_per_s": round(B * layers_done / spec.num_layers / total_dt, 3),
            "sample": f"fp64 oracle {'INT8 ' if kv == 'int8' else ''}append + decode of all {B} sequences for "
                      f"{layers_done} of the "
                      f"{spec.num_layers} layers of the {spec.name} workload ({total_tokens} tokens attended, "
                      f"{kv_bytes} KV bytes); tokens/s scaled to whole {spec.num_layers}-layer steps"}


PREFILL_METRIC = "chunked-prefill paged attention: TFLOP/s of the causal QK^T and PV products (1 GPU)"
ARGMAX_METRIC = "greedy argmax over logit rows: logits GB/s and % of HBM peak (1 GPU)"
MFMA_BF16_PEAK_TFLOPS = 2500.0


def prefill_flops(prefix_lens, chunk_len):
    """Algorithmic flops of one chunk: every (query, key) pair a causal row
    attends (keys 0..pos inclusive) costs 2*64 for q.k and 2*64 for p*v, per
    query head."""
    pairs = sum(int(chunk_len) * (int(p) + 1) + chunk_len * (chunk_len - 1) // 2 for p in prefix_lens)
    return pairs * 32 * 4 * 64, pairs * 32


def cpu_baseline_prefill(case, target_s, kv="bf16"):
    """Time the fp64 oracle's chunked prefill on whole sequences of the workload."""
    import oracle

    total, done, flops = 0.0, 0, 0
    pool_i8 = oracle.quantize_pages_i8(case.k_pool, case.v_pool) if kv == "int8" else None
    for s in range(case.num_seqs):
        one = lambda a: np.ascontiguousarray(a[s:s + 1])
        kp, vp = case.k_pool.copy(), case.v_pool.copy()
        pool = None if pool_i8 is None else pool_i8.copy()
        t0 = time.perf_counter()
        if kv == "int8":
            _, rc = oracle.prefill_chunk_i8(one(case.q).copy(), one(case.k_chunk), one(case.v_chunk), pool,
                                            one(case.block_tables), one(case.prefix_lens), case.num_pages,
                                            case.theta, case.scale)
        else:
            _, rc = oracle.prefill_chunk(one(case.q).copy(), one(case.k_chunk), one(case.v_chunk), kp, vp,
                                         one(case.block_tables), one(case.prefix_lens), case.num_pages, case.theta,
                                         case.scale)
        total += time.perf_counter() - t0
        assert rc == oracle.OK
        done += 1
        flops += prefill_flops(case.prefix_lens[s:s + 1], case.chunk_len)[0]
        if total >= target_s:
            break
    return {"value": round(flops / total / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "cpu_model": host_cpu_model(), "kind": "oracle", "seconds": round(total, 3),
            "sample": f"fp64 oracle chunked prefill{' into INT8 pages' if kv == 'int8' else ''} (append + causal "
                      f"attention) of {done} of the {case.num_seqs} sequences of the workload ({flops} algorithmic "
                      "flops)"}




TOL_BF16_OUT = (1e-2, 1e-2)  # |gpu - ref| <= atol + rtol |ref| on bf16 outputs


def accuracy_stats(got, ref, tol, checked):
    """Error of the GPU outputs against the fp64 oracle: max_abs_err, max_rel_err (over the
    elements with |ref| >= atol, the others being near-zero averages) and the largest
    |err| / (atol + rtol |ref|), which the tolerance bounds by 1."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(got - ref)
    atol, rtol = tol
    big = np.abs(ref) >= atol
    return {"max_abs_err": float(err.max()),
            "max_rel_err": float((err[big] / np.abs(ref[big])).max()) if big.any() else 0.0,
            "max_err_over_tol": float((err / (atol + rtol * np.abs(ref))).max()),
            "atol": atol, "rtol": rtol, "within_tol": bool((err <= atol + rtol * np.abs(ref)).all()),
            "elements": int(err.size), "checked": checked}


def bf16_bits_to_f64(t):
    """A device bf16 tensor as float64 on the host (exact)."""
    import torch

    bits = t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def decode_accuracy(spec, k_pool, v_pool, rows, layers, call_layer, layer_ids, kv, stream):
    """One more fused call per listed layer, after the timed steps, checked over every sequence
    against the oracle's append + decode of the same inputs: q as it is on the device just before
    the call (each call rotates it in place), the layer's new K/V rows, and the pages drawn for the
    workload (the oracle quantises them itself for INT8 pages; the slot the call appends to is
    rewritten by the oracle's own append before it is read)."""
    import oracle
    import torch

    B = spec.num_seqs
    seqs = np.arange(B)
    gots, refs = [], []
    for l in layer_ids:
        L = layers[l]
        q_dev = L["q"].contiguous().view(torch.int16).cpu().numpy().view(np.uint16).copy()
        call_layer(l)
        torch.cuda.synchronize()
        got = bf16_bits_to_f64(L["out"])
        kp, vp, bt, _, kn, vn, lens, npg = host_case(spec, k_pool, v_pool, rows, l, seqs)
        q = q_dev[seqs].copy()
        if kv == "int8":
            pool = oracle.quantize_pages_i8(kp, vp)
            assert oracle.append_kv_rope_i8(q, kn, vn, pool, bt, lens, npg, spec.theta) == oracle.OK
            ref, rc = oracle.decode_gqa_i8(q, pool, bt, lens, npg, spec.scale)
        else:
            assert oracle.append_kv_rope(q, kn, vn, kp, vp, bt, lens, npg, spec.theta) == oracle.OK
            ref, rc = oracle.decode_gqa(q, kp, vp, bt, lens, npg, spec.scale)
        assert rc == oracle.OK
        gots.append(got)
        refs.append(ref)
    return accuracy_stats(np.stack(gots), np.stack(refs), TOL_BF16_OUT,
                          f"every sequence of layer(s) {list(layer_ids)}, all 32 heads x 64 dims, bf16 out")


def timed_steps(fn, steps, warmup, torch, stream):
    """Mean ms per step over `steps` back-to-back steps between two events, after warm_up."""
    warm = warm_up(fn, torch, warmup)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(steps):
        fn()
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps, warm


def cold_steps(fn, n, torch, stream, device):
    """Median ms of n steps, each preceded (outside its events) by a 512 MiB write that evicts the
    256 MB MALL, so the step starts from HBM."""
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=device)
    cold = []
    for i in range(n):
        flush.fill_(i & 0xFF)
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        torch.cuda.synchronize()
        cold.append(a.elapsed_time(b))
    del flush
    return float(np.median(cold))


def run_decode(name, kv, args, torch, binding, device, *, headline, cpu_seconds):
    """Time one decode workload (fused append + decode per layer) and check it against the oracle."""
    spec, k_pool, v_pool, layers, lens, rows = build_workload(name, device)
    table = binding.rope_table(2048 + 64, spec.theta, device)
    ws = binding.decode_workspace(spec.num_seqs, spec.max_blocks, device)
    stream = torch.cuda.current_stream()
    i8 = kv == "int8"
    pool = None
    if i8:
        pool = binding.i8_pool(spec.num_pages, device)
        binding.quantize_pages_i8(pool, k_pool, v_pool)
        torch.cuda.synchronize()

    def call_layer(l, order=None):
        L = layers[l]
        if i8:
            binding.append_decode_gqa_i8(L["out"], L["q"], L["k_new"], L["v_new"], pool, L["bt"], lens, table,
                                         spec.scale, workspace=ws, dispatch_order=order, stream=stream)
        else:
            binding.append_decode_gqa(L["out"], L["q"], L["k_new"], L["v_new"], k_pool, v_pool, L["bt"], lens,
                                      table, spec.scale, workspace=ws, dispatch_order=order, stream=stream)

    # A batch whose workgroups outnumber the 512 that stay resident on the GPU (2 per CU) is
    # dispatched longest first, from an order computed on the device from the device-resident
    # lengths once per step (pa_order_by_length, inside the timed step) and read by every
    # layer's launch; a smaller batch starts all its workgroups at once and runs in slot order.
    # The order deals the ranked sequences in runs from the long and the short end (ORDER_RUNS,
    # measured per page format on four seeded ragged batches).
    parts = -(-spec.max_blocks * 16 // binding.decode_partition_tokens())
    use_order = spec.num_seqs * 8 * parts > RESIDENT_DECODE_WGS
    order_buf = torch.empty(spec.num_seqs, dtype=torch.int32, device=device)
    runs = ORDER_RUNS[kv]

    def make_order():
        return (binding.order_by_length(lens, spec.max_blocks, order_buf, *runs, stream=stream)
                if use_order else None)

    def step_fused(order=None):
        for l in range(spec.num_layers):
            call_layer(l, order)

    def step_main():
        step_fused(make_order())

    def step_separate():
        order = make_order()
        for L in layers:
            if i8:
                binding.append_kv_rope_i8(L["q"], L["k_new"], L["v_new"], pool, L["bt"], lens, table, stream=stream)
                binding.decode_gqa_i8(L["out"], L["q"], pool, L["bt"], lens, spec.scale, workspace=ws,
                                      dispatch_order=order, stream=stream)
            else:
                binding.append_kv_rope(L["q"], L["k_new"], L["v_new"], k_pool, v_pool, L["bt"], lens, table,
                                       stream=stream)
                binding.decode_gqa(L["out"], L["q"], k_pool, v_pool, L["bt"], lens, spec.scale, workspace=ws,
                                   dispatch_order=order, stream=stream)

    # a secondary one-layer workload takes 200 timed steps (a step is ~10 us)
    steps = max(args.steps, 200) if spec.num_layers == 1 and not headline else args.steps
    separate = args.path == "separate"
    step = step_separate if separate else step_main
    ms, warm = timed_steps(step, steps, args.warmup, torch, stream)
    n_pass = max(3, args.steps // 2)
    other_ms = None
    if headline:
        other_ms = timed_steps(step_main if separate else step_separate, max(3, steps // 2), 2, torch, stream)[0]

    # Kernel duration for the roofline.  With the fused path in slot order the timed region
    # above is nothing but the fused kernel, num_layers launches per step back to back on the
    # launch stream, so its mean per launch (gaps included) is ms / num_layers.  Otherwise (the
    # step also computes its order, or runs the separate calls) the fused kernel is timed the
    # same way in a pass of its own, with the order computed once before it.
    fixed_order = make_order()
    dec_ms_mean = ms / spec.num_layers if not (separate or use_order) else \
        timed_steps(lambda: step_fused(fixed_order), n_pass, 1, torch, stream)[0] / spec.num_layers
    # Median per launch: one event pair per step of a further pass (steps of many launches
    # only, where the events' own cost is small against the step).
    seq_ms = []
    if headline and spec.num_layers > 1:
        for _ in range(n_pass):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            step_fused(fixed_order)
            b.record(stream)
            torch.cuda.synchronize()
            seq_ms.append(a.elapsed_time(b))

    # Ordered batches, for comparison: the same fused step in slot order (no order), and with
    # the host's longest-first order (dispatch_order from pa_dispatch_order_longest_first, the
    # host sort inside every timed step; the launch arguments take at most 1024 (sequence,
    # partition) items).
    slot_ms = lf_ms = None
    if use_order:
        slot_ms = timed_steps(step_fused, n_pass, None, torch, stream)[0]
        if spec.num_seqs * parts <= 1024:
            lf_ms = timed_steps(lambda: step_fused(binding.dispatch_order_longest_first(spec.context_lens)), n_pass,
                                None, torch, stream)[0]

    # Cold runs for workloads whose K/V fit in the 256 MB MALL (Infinity Cache).
    kv_step = spec.kv_bytes() // 2048 * KV_TOKEN_BYTES[kv]
    cold_ms = cold_steps(step, max(5, args.steps // 2), torch, stream, device) if kv_step < (512 << 20) else None

    kv_launch = kv_step // spec.num_layers
    gbps = kv_step / (ms * 1e-3) / 1e9
    dec_gbps = kv_launch / (dec_ms_mean * 1e-3) / 1e9
    sfx = "_i8" if i8 else ""
    res = {
        "ms_per_step": round(ms, 5), "value": round(gbps, 2), "unit": "GB/s",
        "tokens_per_s": round(spec.num_seqs / (ms * 1e-3), 1),
        "pct_hbm_peak": round(100.0 * gbps / HBM_PEAK_GBPS, 2), "warmup": warm, "steps": steps,
        "config": {"workload": spec.name, "num_seqs": spec.num_seqs, "context_len": int(spec.context_lens.max()),
                   "mean_context_len": float(spec.context_lens.mean()), "layers": spec.num_layers,
                   "q_heads": 32, "kv_heads": 8, "head_dim": 64, "page_size": 16, "num_pages": spec.num_pages,
                   "kv_format": kv, "kv_bytes_per_token_layer": KV_TOKEN_BYTES[kv],
                   "step": ("per layer: pa_append_decode_gqa%s (append + RoPE + decode, one launch)" % sfx
                            if not separate else
                            "per layer: pa_append_kv_rope%s then pa_decode_gqa%s" % (sfx, sfx)),
                   "decode_partition_tokens": binding.decode_partition_tokens(),
                   "dispatch": (f"longest first, dealt in runs of {runs[0]} long and {runs[1]} short sequences: "
                                "pa_order_by_length on the device once per step (in the timed step), its order "
                                "passed to every layer's launch" if use_order else "slot order")},
        "kv_bytes_per_step": kv_step,
        "roofline": {"bound": "hbm",
                     "kernel": ("k_decode_paged_i8<8,true,nt> (pa_append_decode_gqa_i8)" if i8 else
                                "k_decode_paged<8,true,rows> (pa_append_decode_gqa)"),
                     "achieved": round(dec_gbps, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(dec_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic(kv) if name == "batch64" else None,
                     "bytes_per_launch": kv_launch, "mean_launch_us": round(dec_ms_mean * 1e3, 2)},
    }
    if headline:
        res[("separate_calls_ms_per_step" if not separate else "fused_ms_per_step")] = round(other_ms, 5)
        res["roofline"]["median_launch_us"] = (round(float(np.median(seq_ms)) / spec.num_layers * 1e3, 2)
                                               if seq_ms else None)
        # The same bytes per launch read as one contiguous stream by the plain read probe, from
        # the same pools, a different chunk per launch: the read bandwidth this GPU reaches here.
        ceil_gbps, ceil_us, ceil_chunks = stream_read_ceiling([pool] if i8 else [k_pool, v_pool], kv_launch,
                                                              spec.num_layers, n_pass, torch, binding, device, stream)
        res["roofline"]["stream_read"] = (None if ceil_gbps is None else
                                          {"kernel": "k_stream_read (pa_probe_stream_read), same bytes per launch",
                                           "achieved": round(ceil_gbps, 2), "unit": "GB/s",
                                           "mean_launch_us": round(ceil_us, 2),
                                           "distinct_chunks_per_step": ceil_chunks,
                                           "frac_of_peak": round(ceil_gbps / HBM_PEAK_GBPS, 4),
                                           "decode_frac_of_stream_read": round(dec_gbps / ceil_gbps, 4)})
    def order_figure(m, note):
        return {"ms_per_step": round(m, 5), "value": round(kv_step / (m * 1e-3) / 1e9, 2), "unit": "GB/s",
                "tokens_per_s": round(spec.num_seqs / (m * 1e-3), 1),
                "mean_launch_us": round(m / spec.num_layers * 1e3, 2),
                "frac": round(kv_launch / (m / spec.num_layers * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4), "note": note}

    if slot_ms is not None:
        res["slot_order"] = order_figure(slot_ms, "the fused step without an order: workgroups dealt in batch order")
    if lf_ms is not None:
        res["longest_first"] = order_figure(lf_ms, "fused step with a host dispatch_order = sequences by length, "
                                                   "longest first; the host sort (pa_dispatch_order_longest_first) "
                                                   "runs inside every timed step")
    if cold_ms is not None:
        res["cold"] = {"ms_per_step": round(cold_ms, 5), "value": round(kv_step / (cold_ms * 1e-3) / 1e9, 2),
                       "unit": "GB/s", "pct_hbm_peak": round(100.0 * kv_step / (cold_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
                       "mean_launch_us": round(cold_ms / spec.num_layers * 1e3, 2),
                       "note": "median of steps each preceded (outside its events) by a 512 MiB write that evicts "
                               "the MALL; the main figures are warm"}
    if not args.no_accuracy:
        acc_layers = [0, spec.num_layers - 1] if spec.num_layers > 1 else [0]
        res["accuracy"] = decode_accuracy(spec, k_pool, v_pool, rows, layers, lambda l: call_layer(l, make_order()),
                                          acc_layers, kv, stream)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(spec, k_pool, v_pool, rows, cpu_seconds, kv)
    del spec, k_pool, v_pool, layers, pool, ws
    torch.cuda.empty_cache()
    return res


def run_prefill(args, torch, binding, device, *, cpu_seconds, kv="bf16"):
    """One step = one pa_prefill_chunk call: append the 4 x 512 chunk rows
    (K rotated into pages, q rotated in place), then causal MFMA attention of
    every chunk row over its 1536 + i + 1 keys.  kv="int8": pa_prefill_chunk_i8
    over an INT8 pool quantised from the same pages before timing."""
    from paged_kv_gqa_append_amd import workloads as W

    c = W.prefill_config()

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)

    q, kc, vc, kp, vp = up(c.q), up(c.k_chunk), up(c.v_chunk), up(c.k_pool), up(c.v_pool)
    bt = torch.from_numpy(c.block_tables).to(device)
    prefix = torch.from_numpy(c.prefix_lens).to(device)
    out = torch.empty_like(q)
    table = binding.rope_table(2048 + 64, c.theta, device)
    stream = torch.cuda.current_stream()

    pool = None
    if kv == "int8":
        pool = binding.i8_pool(c.num_pages, device)
        binding.quantize_pages_i8(pool, kp, vp)
        torch.cuda.synchronize()

    # q is rotated in place by every call (a norm-preserving rotation, so its
    # values stay N(0,1)-like); the chunk rows are re-appended at the same slots.
    def step():
        if pool is not None:
            binding.prefill_chunk_i8(out, q, kc, vc, pool, bt, prefix, table, c.scale, stream=stream)
        else:
            binding.prefill_chunk(out, q, kc, vc, kp, vp, bt, prefix, table, c.scale, stream=stream)

    warm = warm_up(step, torch, args.warmup)
    calls = []
    for _ in range(args.steps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        step()
        b.record(stream)
        calls.append((a, b))
    torch.cuda.synchronize()
    per_call = np.array([a.elapsed_time(b) for a, b in calls])
    ms = float(per_call.mean())
    flops, n_exp = prefill_flops(c.prefix_lens, c.chunk_len)
    tflops = flops / (ms * 1e-3) / 1e12
    res = {
        "ms_per_step": round(ms, 5), "value": round(tflops, 2), "unit": "TFLOP/s", "warmup": warm,
        "steps": args.steps,
        "config": {"workload": "chunked_prefill", "num_seqs": c.num_seqs, "prefix_len": int(c.prefix_lens[0]),
                   "chunk_len": c.chunk_len, "layers": 1, "q_heads": 32, "kv_heads": 8, "head_dim": 64,
                   "page_size": 16, "num_pages": c.num_pages, "causal": "inclusive", "kv_format": kv,
                   "step": ("pa_prefill_chunk_i8 (chunk quantised into INT8 pages + RoPE, then causal attention "
                            "over the INT8 pages on f16 MFMA, weights as hi + lo halves)" if pool is not None else
                            "pa_prefill_chunk (chunk append + RoPE, then causal paged attention on MFMA)")},
        "median_ms_per_step": round(float(np.median(per_call)), 5),
        "tokens_per_s": round(c.num_seqs * c.chunk_len / (ms * 1e-3), 1),
        "flops_per_step": flops, "exp_per_step": n_exp,
        "roofline": {"bound": "mfma",
                     "kernel": ("k_append_rope_i8 (prefix mode) + k_prefill_attn_i8, one call; peak of dense f16 MFMA"
                                if pool is not None else "k_append_rope (prefix mode) + k_prefill_attn, one call"),
                     "achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                     "flops_per_launch": flops, "mean_launch_us": round(ms * 1e3, 2)},
    }
    if not args.no_accuracy:
        # one more call; every row of every sequence against the oracle's prefill of the same
        # inputs (q as it is before the call, the drawn pages and chunk rows)
        import oracle

        q_before = q.contiguous().view(torch.int16).cpu().numpy().view(np.uint16).copy()
        step()
        torch.cuda.synchronize()
        got = bf16_bits_to_f64(out)
        refs = []
        pool_host = oracle.quantize_pages_i8(c.k_pool, c.v_pool) if pool is not None else None
        for s in range(c.num_seqs):
            one = lambda a: np.ascontiguousarray(a[s:s + 1])
            if pool_host is not None:
                ref, rc = oracle.prefill_chunk_i8(one(q_before).copy(), one(c.k_chunk), one(c.v_chunk),
                                                  pool_host.copy(), one(c.block_tables), one(c.prefix_lens),
                                                  c.num_pages, c.theta, c.scale)
            else:
                ref, rc = oracle.prefill_chunk(one(q_before).copy(), one(c.k_chunk), one(c.v_chunk),
                                               c.k_pool.copy(), c.v_pool.copy(), one(c.block_tables),
                                               one(c.prefix_lens), c.num_pages, c.theta, c.scale)
            assert rc == oracle.OK
            refs.append(ref[0])
        res["accuracy"] = accuracy_stats(got, np.stack(refs), TOL_BF16_OUT,
                                         f"all {c.num_seqs} x {c.chunk_len} rows, 32 heads x 64 dims, bf16 out")
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_prefill(c, cpu_seconds, kv)
    del pool
    return res


def run_argmax(args, torch, binding, device, *, cpu_seconds):
    """One step = 16 pa_argmax calls over 64 rows of the 128,256-entry Llama 3.2 vocabulary (bf16
    logits ~N(0,1)): the greedy choices of 16 batch-64 decode steps.  Warm: every call reads the
    same 16 MB of logits (they stay in the 256 MB MALL).  Cold (the roofline): the calls rotate
    over 40 distinct 16 MB buffers (656 MB), so each call reads its logits from HBM."""
    from paged_kv_gqa_append_amd import workloads as W

    rows, vocab = 64, W.VOCAB_SIZE
    host = W.f32_to_bf16_bits(W.argmax_logits(5, rows, vocab, specials=False))
    logits = torch.from_numpy(host.view(np.int16)).view(torch.bfloat16).to(device)
    n_bufs = 40
    bufs = [logits.clone() for _ in range(n_bufs)]
    out = torch.empty(rows, dtype=torch.int32, device=device)
    ws = binding.argmax_workspace(rows, vocab, torch.bfloat16, device)
    stream = torch.cuda.current_stream()
    calls_per_step = 16
    nbytes = rows * vocab * 2

    def step_warm():
        for _ in range(calls_per_step):
            binding.argmax(out, logits, workspace=ws, stream=stream)

    nxt = [0]

    def step_cold():
        for _ in range(calls_per_step):
            binding.argmax(out, bufs[nxt[0] % n_bufs], workspace=ws, stream=stream)
            nxt[0] += 1

    ms_w, warm = timed_steps(step_warm, args.steps, args.warmup, torch, stream)
    ms_c, warm_c = timed_steps(step_cold, args.steps, args.warmup, torch, stream)
    us_w = ms_w * 1e3 / calls_per_step
    us_c = ms_c * 1e3 / calls_per_step
    gb_w = nbytes / (us_w * 1e-6) / 1e9
    gb_c = nbytes / (us_c * 1e-6) / 1e9
    res = {
        "ms_per_step": round(ms_c, 5), "value": round(gb_c, 2), "unit": "GB/s", "warmup": warm, "steps": args.steps,
        "config": {"workload": "argmax_batch64", "rows": rows, "vocab": vocab,
                   "step": f"{calls_per_step} x pa_argmax (k_argmax, one launch per call), each on the next of "
                           f"{n_bufs} distinct logit buffers"},
        "us_per_call": round(us_c, 3),
        "roofline": {"bound": "hbm", "kernel": "k_argmax<bf16,vec>, one launch per call, logits from HBM",
                     "achieved": round(gb_c, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gb_c / HBM_PEAK_GBPS, 4), "traffic": measured_traffic("argmax"),
                     "bytes_per_launch": nbytes, "mean_launch_us": round(us_c, 3)},
        "cold_warmup": warm_c,
        "warm": {"ms_per_step": round(ms_w, 5), "value": round(gb_w, 2), "unit": "GB/s", "us_per_call": round(us_w, 3),
                 "frac": round(gb_w / HBM_PEAK_GBPS, 4), "warmup": warm,
                 "note": "every call on the same 16 MB buffer, which stays in the 256 MB MALL; timed first"},
    }
    if not args.no_accuracy:
        import oracle

        got = out.cpu().numpy()
        ref = oracle.argmax(host)
        res["accuracy"] = {"index_mismatches": int((got != ref).sum()), "rows": rows,
                           "checked": "the last timed call's indices against the oracle, exact"}
        assert np.array_equal(got, ref), "argmax differs from the oracle"
    if not args.no_cpu_baseline:
        import oracle

        reps, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < min(cpu_seconds, 5.0):
            oracle.argmax(host)
            reps += 1
        dt = (time.perf_counter() - t0) / reps
        res["cpu_baseline"] = {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1,
                               "cpu_model": host_cpu_model(), "kind": "oracle",
                               "seconds": round(dt * reps, 3),
                               "sample": f"fp64-compare oracle argmax over the same {rows} x {vocab} bf16 rows, "
                                         f"{reps} repetitions, one thread"}
    del bufs, logits
    torch.cuda.empty_cache()
    return res


def line(metric, dtype, res):
    """The contract's fields around one workload's result object."""
    out = {"metric": metric, "value": res["value"], "unit": res["unit"], "n_gpus": 1, "steps": res.get("steps"),
           "warmup": res.get("warmup"), "ms_per_step": res["ms_per_step"], "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": dtype, "data": "synthetic", "config": res["config"]}
    for k, v in res.items():
        if k not in out:
            out[k] = v
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1 "
                                   "(the decode path shards by sequence or KV head with no exchange, "
                                   "but no multi-GPU launcher is built)"}))
        sys.exit(2)
    import torch

    from paged_kv_gqa_append_amd import binding, build

    if not build.is_current():
        build.build()
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    device = torch.device("cuda", 0)
    if args.copy_calibration:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=device).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": 3}), flush=True)
        return
    dec_dtype = "bf16" if args.kv == "bf16" else "int8 K/V, bf16 q/out, fp32 accumulation"
    if args.config == "prefill":
        print(json.dumps(line(PREFILL_METRIC, "bf16" if args.kv == "bf16" else "int8 K/V, f16 MFMA, fp32 accumulation",
                              run_prefill(args, torch, binding, device, cpu_seconds=args.cpu_seconds,
                                          kv=args.kv))), flush=True)
        return
    if args.config == "argmax":
        print(json.dumps(line(ARGMAX_METRIC, "bf16", run_argmax(args, torch, binding, device,
                                                                cpu_seconds=args.cpu_seconds))), flush=True)
        return
    name = args.config or "batch64"
    res = line(METRIC, dec_dtype, run_decode(name, args.kv, args, torch, binding, device, headline=True,
                                             cpu_seconds=args.cpu_seconds))
    if args.config is None:
        # every other workload, each with its own accuracy stamp and bounded oracle baseline
        cs = args.cpu_seconds_secondary
        sec = {}
        for key, wl, kv in [("batch64_int8", "batch64", "int8"), ("batch256_bf16", "batch256", "bf16"),
                            ("batch256_int8", "batch256", "int8"), ("batch8_bf16", "batch8", "bf16"),
                            ("tiny_bf16", "tiny", "bf16")]:
            t0 = time.perf_counter()
            sec[key] = run_decode(wl, kv, args, torch, binding, device, headline=False, cpu_seconds=cs)
            sec[key]["wall_s"] = round(time.perf_counter() - t0, 1)
        t0 = time.perf_counter()
        sec["prefill"] = run_prefill(args, torch, binding, device, cpu_seconds=cs)
        sec["prefill"]["wall_s"] = round(time.perf_counter() - t0, 1)
        t0 = time.perf_counter()
        sec["prefill_int8"] = run_prefill(args, torch, binding, device, cpu_seconds=cs, kv="int8")
        sec["prefill_int8"]["wall_s"] = round(time.perf_counter() - t0, 1)
        t0 = time.perf_counter()
        sec["argmax"] = run_argmax(args, torch, binding, device, cpu_seconds=cs)
        sec["argmax"]["wall_s"] = round(time.perf_counter() - t0, 1)
        res["secondary"] = sec
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
