"""The C ABI's host code under the address and undefined-behaviour
sanitizers (no GPU): gdn_api.cpp is built with g++ for the host only,
linked against stand-ins for the kernel launchers (tests/host/launch_stubs.cpp)
and driven through every status code and argument block by
tests/host/api_driver.cpp.  Any sanitizer report aborts the driver."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST = os.path.join(ROOT, "tests", "host")
ROCM_INCLUDE = "/opt/rocm/include"


def test_api_validation_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir(ROCM_INCLUDE):
        pytest.skip("needs g++ and the ROCm headers")
    exe = str(tmp_path / "api_driver")
    srcs = [os.path.join(ROOT, "gated_deltanet_conv1d_amd", "csrc", "gdn_api.cpp"),
            os.path.join(HOST, "launch_stubs.cpp"), os.path.join(HOST, "api_driver.cpp")]
    flags = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", "-I", ROCM_INCLUDE, "-Wall", "-Wextra",
             "-Wno-unused-parameter", "-Werror"]
    r = subprocess.run([gxx, *flags, *srcs, "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "0 failed" in r.stdout, r.stdout
