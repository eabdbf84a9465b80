"""Host-side checks of the benchmark script: the one-GPU refusal, the traffic
lookup's source-hash guard, and the algorithmic counts its rooflines divide by.
No GPU needed."""
import hashlib
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"]


def _sha(kind):
    h = hashlib.sha256()
    for name in bench.TRAFFIC[kind][0]:
        with open(os.path.join(ROOT, "paged_kv_gqa_append_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def test_traffic_is_reported_only_for_the_recorded_sources(tmp_path):
    for kind, (_, summary) in bench.TRAFFIC.items():
        path = tmp_path / summary
        path.write_text(f"traffic_bytes_per_launch: 123456\nkernel_source_sha256: {_sha(kind)}\n")
        assert bench.measured_traffic(kind, str(tmp_path)) == 123456
        path.write_text("traffic_bytes_per_launch: 123456\nkernel_source_sha256: " + "0" * 64 + "\n")
        assert bench.measured_traffic(kind, str(tmp_path)) is None
        path.unlink()
        assert bench.measured_traffic(kind, str(tmp_path)) is None


def test_prefill_flop_count_matches_the_workload_statement():
    # 4 sequences x (1536 cached + 512-token chunk), causal inclusive: 917,760 (query, key) pairs per
    # (sequence, query head) = 512 x 1536 + 512 x 513 / 2.
    flops, n_exp = bench.prefill_flops([1536] * 4, 512)
    pairs = 4 * 32 * (512 * 1536 + 512 * 513 // 2)
    assert n_exp == pairs == 117_473_280
    assert flops == pairs * 256 == 30_073_159_680
    # a chunk of one token at prefix p attends p + 1 keys
    assert bench.prefill_flops([7], 1) == (8 * 32 * 256, 8 * 32)


def test_int8_bytes_per_token_are_the_tile_share():
    assert bench.KV_TOKEN_BYTES["bf16"] == 8 * 2 * 64 * 2
    assert bench.KV_TOKEN_BYTES["int8"] == 8 * (2 * 64 + 2 * 4) == 1088


def test_host_cpu_model_is_a_string_or_absent():
    m = bench.host_cpu_model()
    assert m is None or (isinstance(m, str) and m)
