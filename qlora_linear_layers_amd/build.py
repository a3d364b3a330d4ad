"""Build the gfx950 HIP library ``libqlora_mi355x.so`` in-tree with hipcc.

Every call compiles from source (a stale library is never reused).  The
device code is built with packed-fp32 instructions disabled and without
fast-math, so IEEE fp32 division, multiplication and denormals are preserved.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB_NAME = "libqlora_mi355x.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
SOURCES = ("codebook.cpp", "quant.hip", "gemm.hip", "lora.hip", "gemv.hip", "merge.hip", "api.cpp")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-fast-math", "-Wno-unused-command-line-argument",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
]


def build(verbose=False):
    srcs = []
    for s in SOURCES:
        p = os.path.join(CSRC, s)
        srcs += (["-x", "hip", p] if s.endswith(".hip") else ["-x", "hip", p])
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC] + FLAGS + srcs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building " + LIB_NAME)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
