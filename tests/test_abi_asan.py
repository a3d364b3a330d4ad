"""The C ABI layer under AddressSanitizer (host code only): the library is
rebuilt with the host half of every translation unit instrumented and the
host-side ABI tests (argument validation, codebook, workspace sizes,
exports) run against it in a child process with the sanitizer runtime
preloaded.  A heap or stack overrun in the host code (descriptor arrays,
table builders, size arithmetic) aborts that process and fails this test."""
import glob
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

from qlora_linear_layers_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
RUNTIME = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
# the sanitizer applies to host code only (device code is never instrumented)
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]

CHILD = """
import sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
from qlora_linear_layers_amd import api
api.LIB_PATH = {lib!r}
import pytest
sys.exit(pytest.main(["-q", "-p", "no:cacheprovider", {test!r}]))
"""


@pytest.mark.slow
@pytest.mark.skipif(not RUNTIME or not os.path.exists(B.HIPCC), reason="no hipcc or clang ASan runtime")
def test_abi_host_under_address_sanitizer():
    with tempfile.TemporaryDirectory() as tmp:
        objs = [os.path.join(tmp, os.path.splitext(s)[0] + ".o") for s in B.SOURCES]

        def compile_one(src, obj):
            return subprocess.run([B.HIPCC] + B.FLAGS + SAN + ["-c", "-x", "hip", os.path.join(B.CSRC, src), "-o", obj],
                                  capture_output=True, text=True)
        with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
            for res in ex.map(compile_one, B.SOURCES, objs):
                assert res.returncode == 0, res.stderr[-2000:]
        lib = os.path.join(tmp, "libqlora_asan.so")
        res = subprocess.run([B.HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
                              "-shared-libasan"] + objs + ["-o", lib], capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-2000:]
        env = dict(os.environ, LD_PRELOAD=RUNTIME[-1], ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
                   LD_LIBRARY_PATH=os.path.dirname(RUNTIME[-1]) + ":" + os.environ.get("LD_LIBRARY_PATH", ""))
        code = CHILD.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=lib,
                            test=os.path.join(ROOT, "tests", "test_abi_host.py"))
        res = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=600)
        assert res.returncode == 0, (res.stdout[-3000:], res.stderr[-3000:])
        assert "passed" in res.stdout
