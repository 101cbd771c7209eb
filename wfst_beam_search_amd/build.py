"""Build the decoder library (HIP for gfx950 + the C ABI) in-tree with hipcc."""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libwfst_mi355x.so")
SOURCES = [os.path.join(HERE, "csrc", "wfst_kernels.hip"), os.path.join(HERE, "csrc", "wfst_noalloc.hip"),
           os.path.join(HERE, "csrc", "wfst_api.cpp")]

FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-shared",
    # every fp32 operation is rounded on its own: no contraction into FMA
    "-ffp-contract=off",
    # no packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    # the kernels' few argument dwords (a Work pointer, step, pass) arrive in
    # SGPRs with the dispatch
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
]


# machine probes (random gathers, dependent chains, atomics, launch floor) for
# bench.py --probe: a library of their own, not part of the decoder
PROBE_LIB = os.path.join(HERE, "libwfst_probe.so")
PROBE_SOURCES = [os.path.join(HERE, "csrc", "wfst_probe.hip")]


def _compile(out: str, sources, verbose: bool) -> None:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = out + f".tmp{os.getpid()}"
    cmd = [hipcc, *FLAGS, "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc"),
           "-o", tmp, *sources]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.check_call(cmd)
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    _compile(LIB, SOURCES, verbose)
    _compile(PROBE_LIB, PROBE_SOURCES, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
