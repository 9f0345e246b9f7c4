"""The C ABI's host code (argument validation, the slot table, the error paths
of create) built with the address and undefined-behaviour sanitizers by the
host C++ compiler, the kernel launchers replaced by host stand-ins, and run
through tests/sanitize/driver.cpp.  CPU only."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.mark.timeout(300)
def test_host_code_under_asan_and_ubsan(tmp_path):
    cxx = shutil.which("g++")
    if cxx is None or not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime_api.h")):
        pytest.skip("g++ or the HIP runtime headers are missing")
    csrc = os.path.join(ROOT, "block_causal_kv_amd", "csrc")
    exe = str(tmp_path / "driver")
    cmd = [cxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(ROCM, "include"),
           os.path.join(csrc, "kvc_api.cpp"), os.path.join(csrc, "slot_table.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "driver.cpp"), os.path.join(ROOT, "tests", "sanitize", "stubs.cpp"),
           "-L" + os.path.join(ROCM, "lib"), "-lamdhip64", "-lrocprofiler-sdk-roctx", "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ)
    # the HIP runtime is not built with the sanitizers: its own allocations at
    # initialisation are not this code's leaks
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:verify_asan_link_order=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=240)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "sanitized host checks passed" in r.stdout
