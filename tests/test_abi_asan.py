"""The host side of the C ABI (csrc/api.cpp: argument validation, overlap
checks, status strings) built with AddressSanitizer, and the ABI tests of
tests/test_abi.py run against that build (no GPU: the kernel launchers are
stubs that return an error, tests/asan/launch_stubs.cpp)."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "nvfp4_quantization_grouped_amd")
OUT = os.path.join(ROOT, "_build", "asan", "libmxq_asan.so")


def _libasan():
    gcc = shutil.which("gcc")
    if not gcc:
        return None
    p = subprocess.run([gcc, "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.fixture(scope="module")
def asan_lib():
    gxx, rt = shutil.which("g++"), _libasan()
    if not gxx or not rt:
        pytest.skip("g++ with libasan is not available")
    os.makedirs(os.path.dirname(OUT), exist_ok=True)
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    # host-only C++ (the ABI layer has no device code): g++ with the HIP headers
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address", "-fno-omit-frame-pointer", "-shared", "-fPIC",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(rocm, "include"), "-I", os.path.join(ROOT, "include"),
           os.path.join(PKG, "csrc", "api.cpp"), os.path.join(ROOT, "tests", "asan", "launch_stubs.cpp"),
           "-o", OUT]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return OUT, rt


def test_abi_tests_pass_under_asan(asan_lib):
    lib, rt = asan_lib
    code = (
        "import sys; sys.path.insert(0, %r)\n"
        "from nvfp4_quantization_grouped_amd import _lib\n"
        "_lib.LIB_PATH = %r\n"
        "import pytest\n"
        "sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', %r]))\n"
    ) % (ROOT, lib, os.path.join(ROOT, "tests", "test_abi.py"))
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:exitcode=86")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out, out[-2000:]
