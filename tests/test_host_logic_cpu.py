"""The C-ABI host code on the CPU, under AddressSanitizer and
UndefinedBehaviorSanitizer: tests/host/echo_host_check.cpp drives libecho's
host code (csrc/echo_api.hip) against recording stand-ins of the kernels and
checks workspace carving, launch arguments, argument errors and wire bytes
for some two thousand configurations, up to the largest message the ABI
takes (no device memory is touched; the workspace is a fake address range)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST = os.path.join(ROOT, "tests", "host")
ROCM_INC = "/opt/rocm/include"


def test_host_logic_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir(ROCM_INC):
        pytest.skip("g++ or the HIP headers are not available")
    exe = str(tmp_path / "echo_host_check")
    sources = [os.path.join(HOST, f) for f in ("echo_api_host.cpp", "echo_host_stubs.cpp", "echo_host_check.cpp")]
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(ROOT, "include"),
           "-I" + os.path.join(ROOT, "error_compensated_bit_echo_amd", "csrc"), "-I" + HOST,
           "-isystem", ROCM_INC, *sources, "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    assert r.stdout.startswith("ok:"), r.stdout
