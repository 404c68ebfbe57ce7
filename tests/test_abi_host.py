"""The C-ABI layer built for the host alone, with AddressSanitizer and
UBSan, against stand-ins for the HIP runtime and the kernel launchers
(tests/abi_host).  It runs every validation case of include/wush.h, checks
that a rejected call makes no HIP call and no launch, and that the
quantizer's launch plan covers every tile and panel for a sweep of shapes.
No GPU and no device code are involved."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCES = [
    os.path.join(ROOT, "mxfp4_activation_amd", "csrc", "wush_abi.cpp"),
    os.path.join(ROOT, "tests", "abi_host", "stubs.cpp"),
    os.path.join(ROOT, "tests", "abi_host", "driver.cpp"),
]


def test_abi_validation_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path / "abi_host")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
           "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-o", exe] + SOURCES
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "abi host checks passed" in r.stdout
