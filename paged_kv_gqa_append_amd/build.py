"""Build libpa.so (HIP kernels + C ABI) for gfx950 in-tree with hipcc."""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libpa.so")
OBJ_DIR = os.path.join(PKG, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-function",
    # keep fp32 math on the scalar-per-lane VALU path
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-ffp-contract=fast", "-fno-fast-math",
]
# Per-source additions.  The MFMA prefill kernel rescales its accumulators
# with VALU multiplies; selecting the VGPR form of the MFMAs keeps them out of
# AGPRs, which otherwise costs a copy of every accumulator each key block.
FILE_FLAGS = {
    "pa_prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
}


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(OBJ_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-I", INCLUDE, "-I", CSRC, "-c", src,
           "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return obj


def build(verbose: bool = False) -> str:
    """Compile every csrc/*.hip and link libpa.so (always recompiles)."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), sources()))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def is_built() -> bool:
    return os.path.exists(LIB)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
