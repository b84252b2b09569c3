"""The host C-ABI layer (argument checks, fan-out arithmetic, workspace
carving, error reporting) built with g++ under AddressSanitizer and
UndefinedBehaviorSanitizer and driven on the CPU by tests/sanitize/
host_abi_driver.cpp: the kernel launchers are stubs, device pointers are
fake addresses the host layer never dereferences. Any sanitizer report
aborts the driver (no recovery), so a clean exit means none was raised."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_abi_under_asan_ubsan(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("needs g++ and the ROCm headers")
    exe = str(tmp_path / "host_abi_driver")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(ROOT, "verify_speculation_cache_amd", "csrc"),
           os.path.join(ROOT, "verify_speculation_cache_amd", "csrc", "ssd_api.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "host_abi_driver.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1", UBSAN_OPTIONS="halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failures" in r.stdout, r.stdout
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr
