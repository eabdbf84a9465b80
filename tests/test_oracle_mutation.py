"""Mutation sweep of the oracle (CPU only): are the pins strong enough?

Each mutant plants one plausible mistake in a copy of oracle/oracle.c (a wrong
head map, a flipped sign, a dropped term, a transposed index, a wrong rounding
rule, an off-by-one position ...), is compiled with the oracle's own flags, and
the pin tests that should notice run against it through the PA_ORACLE_LIB
override.  Every mutant must make at least one pin fail (pytest exit status 1:
a failed assertion, not a crash or a collection error), and the unmutated copy,
built the same way, must pass the same pins.  The pins themselves compare the
oracle with things other than itself (torch SDPA, complex multiplication, the
Hugging Face rotate-half routine, closed forms, exact-rational quantisation,
numpy's argmax), so a mutant that passes would be a mistake they cannot see.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")
T = "tests/test_oracle_"

# (name, text in oracle.c, replacement, occurrences to replace (0 = all), pin files expected to notice)
MUTANTS = [
    ("head map h % 8 instead of h / 4", "h / (O_HQ / O_HKV)", "h % O_HKV", 0,
     [T + "decode.py", T + "prefill.py"]),
    ("rotation: sign of the sine term", "y[i] = x0 * c - x1 * s;", "y[i] = x0 * c + x1 * s;", 1, [T + "rope.py"]),
    ("rotation: frequency exponent -i/64", "-(2.0 * i) / (double)O_D", "-(1.0 * i) / (double)O_D", 1,
     [T + "rope.py"]),
    ("score without the scale", "score_buf[t] = scale * acc;", "score_buf[t] = acc;", 0, [T + "decode.py"]),
    ("V read from the next slot", "const uint16_t *vr = v_pool + pool_index(page, kv_head, (int)(t % O_PS));",
     "const uint16_t *vr = v_pool + pool_index(page, kv_head, (int)((t + 1) % O_PS));", 1, [T + "decode.py"]),
    ("softmax not normalised", "out[d] = o[d] / z;", "out[d] = o[d];", 0, [T + "decode.py"]),
    ("appended token at position L instead of L - 1", "max_blocks, num_pages, L - 1, theta);",
     "max_blocks, num_pages, L, theta);", 1, [T + "rope.py"]),
    ("exclusive causal mask in prefill", "(int64_t)prefix_lens[s] + i + 1, scale, buf);",
     "(int64_t)prefix_lens[s] + i, scale, buf);", 1, [T + "prefill.py"]),
    ("bf16 rounding half up instead of half to even", "double r = rint(ldexp(x, -qexp));",
     "double r = floor(ldexp(x, -qexp) + 0.5);", 1, [T + "bf16.py"]),
    ("pool index with slot and head transposed",
     "(((size_t)page * O_HKV + (size_t)head) * O_PS + (size_t)slot) * O_D",
     "(((size_t)page * O_PS + (size_t)slot) * O_HKV + (size_t)head) * O_D", 1, [T + "decode.py", T + "rope.py"]),
    ("INT8 scale max/128", "float scale = amax / 127.0f;", "float scale = amax / 128.0f;", 1, [T + "i8.py"]),
    ("INT8 codes rounded half away from zero", "c = rintf(v[d] / scale);", "c = roundf(v[d] / scale);", 1,
     [T + "i8.py"]),
    ("INT8 K and V scales swapped on read", "memcpy(&sc, tile + (is_v ? i8_vscale(t) : i8_kscale(t)), 4);",
     "memcpy(&sc, tile + (is_v ? i8_kscale(t) : i8_vscale(t)), 4);", 1, [T + "i8.py"]),
    ("argmax keeps the last maximum", "if (best < 0 || v > bv) {", "if (best < 0 || v >= bv) {", 1,
     [T + "argmax.py"]),
    ("argmax lets NaN through", "if (isnan(v)) continue;", "", 1, [T + "argmax.py"]),
]


def _mutate(text: str, old: str, new: str, count: int) -> str:
    n = text.count(old)
    assert n >= 1, f"mutation site not found: {old!r}"
    if count:
        assert n >= count
        return text.replace(old, new, count)
    return text.replace(old, new)


def _run_pins(lib: str, files) -> subprocess.CompletedProcess:
    env = dict(os.environ, PA_ORACLE_LIB=lib, OMP_NUM_THREADS="2")
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu", *files]
    return subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)


@pytest.mark.slow
def test_every_planted_mistake_fails_a_pin(tmp_path):
    text = open(SRC).read()
    jobs = []
    control = tmp_path / "control.c"
    control.write_text(text)
    every_pin = sorted({f for m in MUTANTS for f in m[4]})
    jobs.append(("unmutated copy", str(control), every_pin))
    for k, (name, old, new, count, files) in enumerate(MUTANTS):
        src = tmp_path / f"mutant{k}.c"
        src.write_text(_mutate(text, old, new, count))
        jobs.append((name, str(src), files))

    def run(job):
        name, src, files = job
        lib = src[:-2] + ".so"
        oracle.compile_c(src, lib)
        return name, _run_pins(lib, files)

    with ThreadPoolExecutor(max_workers=4) as ex:
        results = dict(ex.map(run, jobs))
    ctl = results.pop("unmutated copy")
    assert ctl.returncode == 0, "the unmutated copy must pass its pins:\n" + ctl.stdout[-2000:]
    survivors = [n for n, r in results.items() if r.returncode != 1]
    detail = {n: (r.returncode, r.stdout[-400:]) for n, r in results.items() if r.returncode != 1}
    assert not survivors, f"mutants not caught by a failing pin: {detail}"
    assert len(results) == len(MUTANTS)
