"""The C-ABI code (fa_api.cpp) under AddressSanitizer and UBSan on the host:
every attention entry point is driven with valid and invalid arguments
against stub kernel launchers (tests/sanitized/), so argument validation,
status codes, size arithmetic and the launch/no-launch rule are checked with
memory and undefined-behaviour checks on, without a GPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = "/opt/rocm"


def _build(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime.h")):
        pytest.skip("needs g++ and the ROCm headers")
    exe = str(tmp_path / "abi_sanitized")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
           "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "exact_io_aware_72_amd", "csrc"),
           os.path.join(ROOT, "exact_io_aware_72_amd", "csrc", "fa_api.cpp"),
           os.path.join(ROOT, "tests", "sanitized", "stub_launchers.cpp"),
           os.path.join(ROOT, "tests", "sanitized", "abi_driver.cpp"),
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib"),
           "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and ("asan" in r.stderr.lower() or "ubsan" in r.stderr.lower()):
        pytest.skip("sanitizer runtimes not available: " + r.stderr[-300:])
    assert r.returncode == 0, r.stderr[-3000:]
    return exe


def test_entry_points_under_asan_and_ubsan(tmp_path):
    exe = _build(tmp_path)
    env = dict(os.environ)
    # The HIP runtime library keeps allocations alive until exit by design.
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1"
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-3000:]
    assert "ok: 0 failure(s)" in r.stdout
