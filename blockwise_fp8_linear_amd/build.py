"""Build libfp8blk.so and the measurement probe libfp8probe.so (gfx950 only)
in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfp8blk.so")
SOURCES = ["quant.hip", "gemm.hip", "gemm_mx.hip", "scratch.hip", "plan.cpp", "api.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-function",
    # the direct-to-LDS loads set M0 inside their inline assembly on purpose
    "-Wno-inline-asm",
    # keep the compiler from forming packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


# The measurement probe (not the hot path): include/fp8probe.h.
PROBE_LIB = os.path.join(HERE, "libfp8probe.so")
PROBE_SOURCES = ["probe.hip"]


def _compile(sources: list[str], out: str, extra: list[str] | None, verbose: bool) -> str:
    srcs = [os.path.join(CSRC, s) for s in sources]
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, *(extra or []), *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, out)
    return out


def build(extra: list[str] | None = None, out: str = LIB, verbose: bool = False) -> str:
    _compile(PROBE_SOURCES, PROBE_LIB, extra, verbose)
    return _compile(SOURCES, out, extra, verbose)


if __name__ == "__main__":
    print(build(sys.argv[1:], verbose=True))
