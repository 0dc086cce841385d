"""Build ``libhr.so`` (the C-ABI library and its gfx950 kernels) in-tree.

Run ``python -m message_fp16_all_amd.build`` or call ``build()``.  The
library is compiled by hipcc for gfx950 only, without fast-math, and with
packed FP32 instruction selection switched off (the kernels do binary16
arithmetic; nothing in them wants packed FP32).
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libhr.so")
SOURCES = [os.path.join(CSRC, f) for f in ("fold.hip", "exchange.hip", "admit.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-fvisibility=hidden",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # kernels receive their first five arguments in SGPRs (the per-rank
    # exchange kernels put what their first loads need there)
    "-mllvm", "-amdgpu-kernarg-preload-count=5",
    "-I", INCLUDE,
    "-Wl,-rpath,/opt/rocm/lib",
]


def build(verbose: bool = False, defines=(), lib: str = LIB) -> str:
    """Compile every source into ``lib`` (``message_fp16_all_amd/libhr.so``
    by default); ``defines`` are extra preprocessor macros (the diagnostic
    timeline build uses HR_TIMELINE)."""
    tmp = lib + ".tmp"
    cmd = [HIPCC, *FLAGS, *(f"-D{d}" for d in defines), *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
