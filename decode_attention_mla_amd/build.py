"""Build the gfx950 shared libraries in-tree with hipcc: ``libmla_decode.so``
(the decode path) and ``libmla_bench.so`` (the benchmark's measurement
kernels).

Run as ``python -m decode_attention_mla_amd.build`` (or via
``__graft_entry__.build()``).  hipcc cross-compiles for gfx950 without a GPU.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_NAME = "libmla_decode.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
SOURCES = ["mla_decode.hip", "planner.cpp"]
BENCH_LIB_PATH = os.path.join(PKG_DIR, "libmla_bench.so")
BENCH_SOURCES = ["mla_bench.hip"]

# Packed-FP32 VALU forms are kept out of the generated code (see the build
# notes); hipcc's host pass warns that it does not know the feature.  The
# first 16 dwords of every kernel's arguments are preloaded into SGPRs by the
# dispatcher (the split-KV and combine kernels put the values they read
# first there), which saves each workgroup a round trip before its first load.
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-mllvm", "-amdgpu-kernarg-preload-count=16",
             "-Wno-unused-command-line-argument"]


def hipcc_path() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the gfx950 library cannot be built")


def _compile(srcs, out, verbose, extra_flags) -> None:
    tmp = out + ".tmp"
    cmd = [hipcc_path(), *HIP_FLAGS, *(extra_flags or []), "-I", os.path.join(PKG_DIR, "..", "include"),
           *[os.path.join(CSRC, s) for s in srcs], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(line for line in (res.stdout + res.stderr).splitlines()
                     if "packed-fp32-ops" not in line and line.strip())
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{msgs}")
    if verbose and msgs:
        print(msgs, flush=True)
    os.replace(tmp, out)


def build(verbose: bool = False, extra_flags=None) -> str:
    """Compile both libraries (always recompiles); returns the decode library's path."""
    _compile(SOURCES, LIB_PATH, verbose, extra_flags)
    _compile(BENCH_SOURCES, BENCH_LIB_PATH, verbose, extra_flags)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
