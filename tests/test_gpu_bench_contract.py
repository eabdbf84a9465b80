"""The benchmark's one JSON line, from a real run on the GPU: the fields the
round-end driver reads (metric, value, unit, n_gpus, steps, warmup,
ms_per_step, higher_is_better, scaling, vs_baseline, dtype, data, config with
its workload), the roofline object (bound, achieved, peak, unit, frac =
achieved / peak, traffic, and the read ceiling beside it) and the CPU
baseline (the oracle, its thread count and sample), and the accuracy stamp
(the outputs of a call made after the timed steps against the oracle: within
the bf16 tolerance, or no argmax index differing).  The tiny decode workload,
the prefill and the argmax line run in child processes, one after the other,
with short step counts."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                       timeout=240, cwd=ROOT)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    return json.loads(r.stdout.strip().splitlines()[-1])


def check_common(line, steps, unit, bound):
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in line, key
    assert line["n_gpus"] == 1 and line["steps"] == steps and line["unit"] == unit
    assert line["value"] > 0 and line["ms_per_step"] > 0 and line["higher_is_better"] is True
    assert line["vs_baseline"] is None and line["data"] == "synthetic"
    assert isinstance(line["config"]["workload"], str) and line["config"]["workload"]
    r = line["roofline"]
    assert r["bound"] == bound and r["achieved"] > 0 and r["peak"] > 0
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    assert "traffic" in r
    cb = line["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1 and cb["sample"]
    acc = line["accuracy"]
    if "index_mismatches" in acc:
        assert acc["index_mismatches"] == 0
    else:
        assert acc["within_tol"] and acc["max_err_over_tol"] <= 1.0 and acc["elements"] > 0


def test_decode_line():
    print("bench contract: tiny decode", flush=True)
    line = run_bench("--config", "tiny", "--steps", "5", "--warmup", "3", "--cpu-seconds", "1")
    check_common(line, 5, "GB/s", "hbm")
    assert line["config"]["workload"] == "tiny_decode"
    sr = line["roofline"]["stream_read"]
    assert sr["achieved"] > 0 and sr["mean_launch_us"] > 0 and sr["distinct_chunks_per_step"] >= 1
    ratio = line["roofline"]["achieved"] / sr["achieved"]  # both rounded in the line
    assert abs(sr["decode_frac_of_stream_read"] - ratio) <= 1e-2 * ratio + 1e-4


def test_argmax_line():
    print("bench contract: argmax", flush=True)
    line = run_bench("--config", "argmax", "--steps", "3", "--warmup", "2", "--cpu-seconds", "1")
    check_common(line, 3, "GB/s", "hbm")
    # the roofline is the cold figure (logits from HBM); the warm one is beside it
    assert line["value"] == line["roofline"]["achieved"] and line["warm"]["value"] > 0


def test_prefill_line():
    print("bench contract: prefill", flush=True)
    line = run_bench("--config", "prefill", "--steps", "3", "--warmup", "2", "--cpu-seconds", "1")
    check_common(line, 3, "TFLOP/s", "mfma")
    assert line["accuracy"]["elements"] == 4 * 512 * 32 * 64


def test_prefill_int8_line():
    print("bench contract: prefill over INT8 pages", flush=True)
    line = run_bench("--config", "prefill", "--kv", "int8", "--steps", "3", "--warmup", "2", "--cpu-seconds", "1")
    check_common(line, 3, "TFLOP/s", "mfma")
    assert line["config"]["kv_format"] == "int8"
    assert line["accuracy"]["elements"] == 4 * 512 * 32 * 64
