#!/usr/bin/env python3
"""Benchmark: paged GQA decode with KV append on one MI355X.

Default workload (one "step"): 64 sequences at context 2048 (2047 cached
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
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBPS = 8000.0
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
    ap.add_argument("--config", default="batch64",
                    choices=["batch64", "batch256", "batch8", "tiny", "prefill", "argmax"],
                    help="decode workloads, 'prefill': 4 x (1536 cached + 512-token chunk) chunked prefill, or "
                         "'argmax': greedy choice over 64 x 128,256 bf16 logits")
    ap.add_argument("--path", default="fused", choices=["fused", "separate"])
    ap.add_argument("--kv", default="bf16", choices=["bf16", "int8"],
                    help="K/V page format: bf16 pools, or INT8 tiles (codes + one fp32 scale per token and head), "
                         "quantised on the device from the same bf16 pages before timing")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (3 times): under rocprofv3 --pmc its FETCH_SIZE / "
                         "WRITE_SIZE give the factor that scales those counters to bytes")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU work of the oracle sample")
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


def cpu_baseline(spec, k_pool, v_pool, rows, target_s, kv="bf16"):
    """Time the fp64 oracle's append + decode on whole layers of the workload (host cores).

    For INT8 pages the oracle quantises the layer's bf16 pages itself (untimed)
    and its INT8 append + decode are timed."""
    import oracle
    import torch

    # sample: whole layers of the workload, in order, until the CPU budget is spent
    def host_case(layer, seqs):
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

    def run(seqs, layer):
        kp, vp, bt, q, kn, vn, lens, npg = host_case(layer, seqs)
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
MFMA_BF16_PEAK_TFLOPS = 2500.0


def prefill_flops(prefix_lens, chunk_len):
    """Algorithmic flops of one chunk: every (query, key) pair a causal row
    attends (keys 0..pos inclusive) costs 2*64 for q.k and 2*64 for p*v, per
    query head."""
    pairs = sum(int(chunk_len) * (int(p) + 1) + chunk_len * (chunk_len - 1) // 2 for p in prefix_lens)
    return pairs * 32 * 4 * 64, pairs * 32


def cpu_baseline_prefill(case, target_s):
    """Time the fp64 oracle's chunked prefill on whole sequences of the workload."""
    import oracle

    total, done, flops = 0.0, 0, 0
    for s in range(case.num_seqs):
        one = lambda a: np.ascontiguousarray(a[s:s + 1])
        kp, vp = case.k_pool.copy(), case.v_pool.copy()
        t0 = time.perf_counter()
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
            "sample": f"fp64 oracle chunked prefill (append + causal attention) of {done} of the {case.num_seqs} "
                      f"sequences of the workload ({flops} algorithmic flops)"}


def main_prefill(args, torch, binding, device):
    """One step = one pa_prefill_chunk call: append the 4 x 512 chunk rows
    (K rotated into pages, q rotated in place), then causal MFMA attention of
    every chunk row over its 1536 + i + 1 keys."""
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

    # q is rotated in place by every call (a norm-preserving rotation, so its
    # values stay N(0,1)-like); the chunk rows are re-appended at the same slots.
    def step():
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
        "metric": PREFILL_METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": warm, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "chunked_prefill", "num_seqs": c.num_seqs, "prefix_len": int(c.prefix_lens[0]),
                   "chunk_len": c.chunk_len, "layers": 1, "q_heads": 32, "kv_heads": 8, "head_dim": 64,
                   "page_size": 16, "num_pages": c.num_pages, "causal": "inclusive",
                   "step": "pa_prefill_chunk (chunk append + RoPE, then causal paged attention on MFMA)"},
        "median_ms_per_step": round(float(np.median(per_call)), 5),
        "tokens_per_s": round(c.num_seqs * c.chunk_len / (ms * 1e-3), 1),
        "flops_per_step": flops, "exp_per_step": n_exp,
        "roofline": {"bound": "mfma", "kernel": "k_append_rope (prefix mode) + k_prefill_attn, one call",
                     "achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                     "flops_per_launch": flops, "mean_launch_us": round(ms * 1e3, 2)},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_prefill(c, args.cpu_seconds)
    print(json.dumps(res), flush=True)


ARGMAX_METRIC = "greedy argmax over logit rows: logits GB/s and % of HBM peak (1 GPU)"


def main_argmax(args, torch, binding, device):
    """One step = one pa_argmax call over 64 rows of the 128,256-entry Llama 3.2
    vocabulary (bf16 logits ~N(0,1)): the greedy choice of a batch-64 decode step."""
    import oracle
    from paged_kv_gqa_append_amd import workloads as W

    rows, vocab = 64, W.VOCAB_SIZE
    host = W.f32_to_bf16_bits(W.argmax_logits(5, rows, vocab, specials=False))
    logits = torch.from_numpy(host.view(np.int16)).view(torch.bfloat16).to(device)
    out = torch.empty(rows, dtype=torch.int32, device=device)
    ws = binding.argmax_workspace(rows, vocab, torch.bfloat16, device)
    stream = torch.cuda.current_stream()
    calls_per_step = 16

    def step():
        for _ in range(calls_per_step):
            binding.argmax(out, logits, workspace=ws, stream=stream)

    warm = warm_up(step, torch, args.warmup)
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(args.steps):
        step()
    b.record(stream)
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / (args.steps * calls_per_step)
    assert np.array_equal(out.cpu().numpy(), oracle.argmax(host)), "argmax differs from the oracle"
    nbytes = rows * vocab * 2
    gbps = nbytes / (us * 1e-6) / 1e9
    res = {
        "metric": ARGMAX_METRIC, "value": round(gbps, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": warm, "ms_per_step": round(us * calls_per_step * 1e-3, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "argmax_batch64", "rows": rows, "vocab": vocab,
                   "step": f"{calls_per_step} x pa_argmax (k_argmax, one launch per call)"},
        "us_per_call": round(us, 3),
        "roofline": {"bound": "hbm", "kernel": "k_argmax<bf16,vec>, one launch per call",
                     "achieved": round(gbps, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": measured_traffic("argmax"),
                     "bytes_per_launch": nbytes,
                     "mean_launch_us": round(us, 3)},
    }
    if not args.no_cpu_baseline:
        reps, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < min(args.cpu_seconds, 5.0):
            oracle.argmax(host)
            reps += 1
        dt = (time.perf_counter() - t0) / reps
        res["cpu_baseline"] = {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1,
                               "cpu_model": host_cpu_model(), "kind": "oracle",
                               "seconds": round(dt * reps, 3),
                               "sample": f"fp64-compare oracle argmax over the same {rows} x {vocab} bf16 rows, "
                                         f"{reps} repetitions, one thread"}
    print(json.dumps(res), flush=True)


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
    if args.config == "prefill":
        main_prefill(args, torch, binding, device)
        return
    if args.config == "argmax":
        main_argmax(args, torch, binding, device)
        return
    spec, k_pool, v_pool, layers, lens, rows = build_workload(args.config, device)
    table = binding.rope_table(2048 + 64, spec.theta, device)
    ws = binding.decode_workspace(spec.num_seqs, spec.max_blocks, device)
    stream = torch.cuda.current_stream()
    i8 = args.kv == "int8"
    if i8:
        pool = binding.i8_pool(spec.num_pages, device)
        binding.quantize_pages_i8(pool, k_pool, v_pool)
        torch.cuda.synchronize()

    def step_fused(order=None):
        for L in layers:
            if i8:
                binding.append_decode_gqa_i8(L["out"], L["q"], L["k_new"], L["v_new"], pool, L["bt"], lens, table,
                                             spec.scale, workspace=ws, dispatch_order=order, stream=stream)
            else:
                binding.append_decode_gqa(L["out"], L["q"], L["k_new"], L["v_new"], k_pool, v_pool, L["bt"], lens,
                                          table, spec.scale, workspace=ws, dispatch_order=order, stream=stream)

    def step_separate():
        for L in layers:
            if i8:
                binding.append_kv_rope_i8(L["q"], L["k_new"], L["v_new"], pool, L["bt"], lens, table, stream=stream)
                binding.decode_gqa_i8(L["out"], L["q"], pool, L["bt"], lens, spec.scale, workspace=ws,
                                      stream=stream)
            else:
                binding.append_kv_rope(L["q"], L["k_new"], L["v_new"], k_pool, v_pool, L["bt"], lens, table,
                                       stream=stream)
                binding.decode_gqa(L["out"], L["q"], k_pool, v_pool, L["bt"], lens, spec.scale, workspace=ws,
                                   stream=stream)

    def timed(fn, steps, warmup):
        warm = warm_up(fn, torch, warmup)
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for _ in range(steps):
            fn()
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / steps, warm

    step = step_fused if args.path == "fused" else step_separate
    ms, warm = timed(step, args.steps, args.warmup)
    other_ms = timed(step_separate if args.path == "fused" else step_fused, max(3, args.steps // 2), 2)[0]

    # Kernel duration for the roofline.  With the fused path the timed region above is
    # nothing but the fused kernel, num_layers launches per step back to back on the
    # launch stream, so its mean per launch (gaps included) is ms / num_layers.  With the
    # separate path the fused kernel is timed the same way in a pass of its own.
    n_pass = max(3, args.steps // 2)
    if args.path == "fused":
        dec_ms_mean = ms / spec.num_layers
    else:
        dec_ms_mean = timed(step_fused, n_pass, 1)[0] / spec.num_layers
    # Median per launch: one event pair per step of a further pass (steps of many launches
    # only, where the events' own cost is small against the step).
    seq_ms = []
    if spec.num_layers > 1:
        for _ in range(n_pass):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            step_fused()
            b.record(stream)
            torch.cuda.synchronize()
            seq_ms.append(a.elapsed_time(b))

    # Ragged batches: the same fused step with the sequences dispatched longest first (the
    # dispatch_order argument; same results bit for bit), reported beside the slot-order figures.
    # Timed before the cold runs, after the same time-based warmup as the main figures.
    lf_ms = None
    if len(set(spec.context_lens.tolist())) > 1 and spec.num_seqs <= 1024:
        order = binding.dispatch_order_longest_first(spec.context_lens)
        lf_ms = timed(lambda: step_fused(order), n_pass, None)[0]

    # Cold runs for workloads whose K/V fit in the 256 MB MALL (Infinity Cache): before each
    # timed step, outside its events, 512 MiB are written so the step starts from HBM.
    kv_step_bytes = spec.kv_bytes() // 2048 * KV_TOKEN_BYTES[args.kv]
    cold_ms = None
    if kv_step_bytes < (512 << 20):
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=device)
        cold = []
        for i in range(max(5, args.steps // 2)):
            flush.fill_(i & 0xFF)
            torch.cuda.synchronize()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            step()
            b.record(stream)
            torch.cuda.synchronize()
            cold.append(a.elapsed_time(b))
        cold_ms = float(np.median(cold))
        del flush

    kv_step = kv_step_bytes
    kv_launch = kv_step // spec.num_layers
    longest = None
    if lf_ms is not None:
        longest = {"ms_per_step": round(lf_ms, 5), "value": round(kv_step / (lf_ms * 1e-3) / 1e9, 2), "unit": "GB/s",
                   "tokens_per_s": round(spec.num_seqs / (lf_ms * 1e-3), 1),
                   "mean_launch_us": round(lf_ms / spec.num_layers * 1e3, 2),
                   "note": "fused step with dispatch_order = sequences by length, longest first"}
    # The same bytes per launch read as one contiguous stream by the plain read probe, from the
    # same pools, a different chunk per launch: the read bandwidth this GPU reaches at this size.
    ceil_gbps, ceil_us, ceil_chunks = stream_read_ceiling([pool] if i8 else [k_pool, v_pool], kv_launch, spec.num_layers,
                                             n_pass, torch, binding, device, stream)
    gbps = kv_step / (ms * 1e-3) / 1e9
    dec_gbps = kv_launch / (dec_ms_mean * 1e-3) / 1e9
    sfx = "_i8" if i8 else ""
    res = {
        "metric": METRIC, "value": round(gbps, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": warm, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if not i8 else "int8 K/V, bf16 q/out, fp32 accumulation",
        "data": "synthetic",
        "config": {"workload": spec.name, "num_seqs": spec.num_seqs, "context_len": int(spec.context_lens.max()),
                   "mean_context_len": float(spec.context_lens.mean()), "layers": spec.num_layers,
                   "q_heads": 32, "kv_heads": 8, "head_dim": 64, "page_size": 16, "num_pages": spec.num_pages,
                   "kv_format": args.kv, "kv_bytes_per_token_layer": KV_TOKEN_BYTES[args.kv],
                   "step": ("per layer: pa_append_decode_gqa%s (append + RoPE + decode, one launch)" % sfx
                            if args.path == "fused" else
                            "per layer: pa_append_kv_rope%s then pa_decode_gqa%s" % (sfx, sfx)),
                   "decode_partition_tokens": binding.decode_partition_tokens()},
        "tokens_per_s": round(spec.num_seqs / (ms * 1e-3), 1),
        "pct_hbm_peak": round(100.0 * gbps / HBM_PEAK_GBPS, 2),
        "kv_bytes_per_step": kv_step,
        ("separate_calls_ms_per_step" if args.path == "fused" else "fused_ms_per_step"): round(other_ms, 5),
        "roofline": {"bound": "hbm",
                     "kernel": ("k_decode_paged_i8<8,true,nt> (pa_append_decode_gqa_i8)" if i8 else
                                "k_decode_paged<8,true,rows> (pa_append_decode_gqa)"),
                     "achieved": round(dec_gbps, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(dec_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic(args.kv) if args.config == "batch64" else None,
                     "bytes_per_launch": kv_launch, "mean_launch_us": round(dec_ms_mean * 1e3, 2),
                     "median_launch_us": (round(float(np.median(seq_ms)) / spec.num_layers * 1e3, 2)
                                          if seq_ms else None),
                     "stream_read": (None if ceil_gbps is None else
                                     {"kernel": "k_stream_read (pa_probe_stream_read), same bytes per launch",
                                      "achieved": round(ceil_gbps, 2), "unit": "GB/s",
                                      "mean_launch_us": round(ceil_us, 2),
                                      "distinct_chunks_per_step": ceil_chunks,
                                      "frac_of_peak": round(ceil_gbps / HBM_PEAK_GBPS, 4),
                                      "decode_frac_of_stream_read": round(dec_gbps / ceil_gbps, 4)})},
    }
    if longest is not None:
        res["longest_first"] = longest
    if cold_ms is not None:
        res["cold"] = {"ms_per_step": round(cold_ms, 5), "value": round(kv_step / (cold_ms * 1e-3) / 1e9, 2),
                       "unit": "GB/s", "pct_hbm_peak": round(100.0 * kv_step / (cold_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
                       "note": "median of steps each preceded (outside its events) by a 512 MiB write that evicts "
                               "the MALL; the main figures are warm"}
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(spec, k_pool, v_pool, rows, args.cpu_seconds, args.kv)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
