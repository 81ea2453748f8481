"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

csrc/gdr_api.cpp is compiled with g++ (not hipcc: only host code is built here) together with
tests/sanitize/host_check.cpp, which stubs the kernel launchers and the HIP calls the host code makes,
runs valid calls through the whole host path (argument validation, workspace carving, segment plan,
launch order, timing records, the no-allocation entry) and invalid ones that must be rejected before
any launch, and checks that every pointer handed to a launcher lies inside the workspace.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_deltanet_prefill_gdr_amd", "csrc")


def test_host_code_under_asan_and_ubsan(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("g++ or the ROCm headers are missing")
    exe = str(tmp_path / "host_check")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "gdr_api.cpp"), os.path.join(ROOT, "tests", "sanitize", "host_check.cpp"), "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    print(res.stdout, res.stderr)
    assert res.returncode == 0 and "host_check OK" in res.stdout, res.stderr[-4000:]
