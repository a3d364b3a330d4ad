"""Build the gfx950 HIP library ``libqlora_mi355x.so`` in-tree with hipcc.

Every call compiles from source (a stale library is never reused): each source
file becomes an object in parallel, then the objects are linked into the
shared library.  The device code is built with packed-fp32 instructions
disabled and without fast-math, so IEEE fp32 division, multiplication and
denormals are preserved.
"""
import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB_NAME = "libqlora_mi355x.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
SOURCES = ("codebook.cpp", "quant.hip", "gemm.hip", "lora.hip", "gemv.hip", "merge.hip", "api.cpp", "calib.hip")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-fast-math", "-Wno-unused-command-line-argument",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed: " + " ".join(cmd[-3:]))


def build(verbose=False, jobs=None):
    tmpdir = tempfile.mkdtemp(prefix="qlora_build_", dir=HERE)
    try:
        objs = [os.path.join(tmpdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
        cmds = [[HIPCC] + FLAGS + ["-c", "-x", "hip", os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
        with ThreadPoolExecutor(max_workers=jobs or min(len(cmds), os.cpu_count() or 1, 8)) as ex:
            for f in [ex.submit(_run, c, verbose) for c in cmds]:
                f.result()
        tmp = LIB_PATH + ".tmp"
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp], verbose)
        os.replace(tmp, LIB_PATH)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
