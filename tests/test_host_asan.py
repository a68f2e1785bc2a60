"""Host code of the library under AddressSanitizer (CPU, no GPU needed).

The library's host code (argument validation, launch planning, plan
descriptions, overrides, host scalars) is compiled with ASan and linked with
a driver, tests/host/abi_host_paths.cpp, that walks those paths over a sweep
of shapes, short output buffers, malformed overrides and invalid arguments.
The device code is compiled as usual (gfx950, no sanitizer) but never
launched on these paths, so the test runs anywhere hipcc is installed.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from fp8_quantized_linear_amd import build as B  # noqa: E402

pytestmark = pytest.mark.slow

ASAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]


def _tool(name):
    try:
        return B._hipcc() if name == "hipcc" else shutil.which(name)
    except RuntimeError:
        return None


@pytest.mark.skipif(_tool("hipcc") is None or _tool("g++") is None, reason="hipcc or g++ missing")
def test_host_paths_under_address_sanitizer(tmp_path):
    hipcc, gxx = _tool("hipcc"), _tool("g++")
    flags = list(B.HIPCC_FLAGS)

    def compile_one(src):
        obj = str(tmp_path / (src + ".o"))
        cmd = [hipcc, *flags, *ASAN_HOST, "-I", B.CSRC, "-c",
               os.path.join(B.CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        return obj

    with ThreadPoolExecutor(4) as ex:
        objs = list(ex.map(compile_one, B.SOURCES))
    rocm_lib = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(hipcc))), "lib")
    lib = str(tmp_path / "libfql_asan.so")
    r = subprocess.run([gxx, "-shared", "-fsanitize=address", *objs, "-o", lib, "-L", rocm_lib,
                        "-lamdhip64", f"-Wl,-rpath,{rocm_lib}"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    exe = str(tmp_path / "abi_host_paths")
    r = subprocess.run([gxx, "-std=c++17", "-g", "-fsanitize=address", "-fno-omit-frame-pointer",
                        "-I", os.path.join(ROOT, "include"),
                        os.path.join(ROOT, "tests", "host", "abi_host_paths.cpp"), lib, "-o", exe,
                        f"-Wl,-rpath,{tmp_path}", "-L", rocm_lib, "-lamdhip64",
                        f"-Wl,-rpath,{rocm_lib}"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    assert r.returncode == 0 and "host paths done" in r.stdout, (r.stdout[-2000:], r.stderr[-4000:])
