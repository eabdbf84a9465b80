"""The decode partition size is a library constant (2048 tokens) so that a
sequence's output does not depend on the batch; a development switch
(PA_DECODE_PART_PAGES, read once per process) sets it for experiments.  At 8
and 32 pages nearly every sequence of the case spans several partitions, so
the partial results and k_decode_merge carry it: decode and append + decode,
bf16 and INT8 pages, must still meet the oracle's tolerance.  Each size runs
in a child process of its own, one after the other."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.parametrize("pages", [8, 32])
def test_decode_at_other_partition_sizes(pages):
    print(f"partition sweep: {pages} pages", flush=True)
    env = dict(os.environ, PA_DECODE_PART_PAGES=str(pages))
    r = subprocess.run([sys.executable, os.path.join(HERE, "_partition_child.py")], env=env, capture_output=True,
                       text=True, timeout=240)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line == {"partition_tokens": pages * 16, "ok": True}
