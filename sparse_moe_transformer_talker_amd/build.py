"""Build libtalker_moe.so (HIP for gfx950) in the package directory.

Each ``csrc/*.hip`` file is compiled to an object under ``_build/`` at the
repository root (in parallel), then linked into one shared library.  Runs on a
machine without a GPU: hipcc cross-compiles for gfx950.

    python -m sparse_moe_transformer_talker_amd.build
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libtalker_moe.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)

SOURCES = ["route.hip", "permute.hip", "gemm.hip", "decode.hip", "elementwise.hip", "attention.hip", "api.hip"]
HEADERS = ["common.hpp", "kernels.hpp"]

ARCH = "gfx950"
# Packed-fp32 VALU forms are disabled for the device code; hipcc's host pass
# warns that it does not know the feature, which is harmless.
CFLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", INCLUDE, "-I", CSRC]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines() if "is not a recognized feature for this target" not in l)
    if res.returncode != 0:
        raise RuntimeError("command failed (%d): %s\n%s" % (res.returncode, " ".join(cmd), out))
    if verbose and out.strip():
        print(out, flush=True)


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compile every HIP source and link the library; returns its path."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = [os.path.join(BUILD_DIR, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    cmds = [[hipcc, *CFLAGS, "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
    jobs = jobs or min(len(cmds), max(1, min(8, os.cpu_count() or 1)))
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    tmp = LIB_PATH + ".tmp"
    _run([hipcc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
