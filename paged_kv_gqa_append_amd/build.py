"""Build libpa.so (HIP kernels + C ABI) for gfx950 in-tree with hipcc."""
from __future__ import annotations

import glob
import hashlib
import os
import re
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


def digest_inputs():
    """Every file the library is compiled from: the kernel sources, their
    headers and the ABI header."""
    files = sources() + sorted(glob.glob(os.path.join(CSRC, "*.h"))) + [os.path.join(INCLUDE, "pa.h")]
    return files


def source_digest() -> str:
    """sha256 over the library's source files (names and bytes) and the compile
    flags: the build id a library built from this tree carries."""
    h = hashlib.sha256()
    for f in digest_inputs():
        h.update(os.path.relpath(f, ROOT).encode() + b"\0")
        with open(f, "rb") as fh:
            h.update(fh.read())
        h.update(b"\0")
    h.update(repr((FLAGS, sorted(FILE_FLAGS.items()))).encode())
    return h.hexdigest()


def built_digest():
    """The build id inside the built libpa.so (read from the file, not loaded), or None."""
    try:
        with open(LIB, "rb") as fh:
            data = fh.read()
    except OSError:
        return None
    m = re.search(rb"pa-build-id:([0-9a-f]{64})", data)
    return m.group(1).decode() if m else None


def is_current() -> bool:
    """libpa.so exists and was built from the sources now in the tree."""
    return built_digest() == source_digest()


def _compile(src: str, verbose: bool, digest: str) -> str:
    obj = os.path.join(OBJ_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), f'-DPA_BUILD_ID="{digest}"', "-I", INCLUDE,
           "-I", CSRC, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return obj


def build(verbose: bool = False) -> str:
    """Compile every csrc/*.hip and link libpa.so (always recompiles)."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    digest = source_digest()
    with ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, digest), sources()))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def is_built() -> bool:
    """libpa.so exists (whatever it was built from; see is_current)."""
    return os.path.exists(LIB)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
