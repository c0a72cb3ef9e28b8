"""The library's host code (layout building, work-item tables, argument validation) under
AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

tests/native/host_abi_check.cpp is compiled with g++ together with the library's host sources
(layout.cpp, api.cpp; no device code, the kernel launchers are aborting stubs) and run.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_host_code_under_sanitizers(tmp_path):
    exe = str(tmp_path / "host_abi_check")
    csrc = os.path.join(ROOT, "all_gather_placement_amd", "csrc")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "native", "host_abi_check.cpp"),
           os.path.join(csrc, "layout.cpp"), os.path.join(csrc, "api.cpp"),
           "-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib", "-lamdhip64", "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, timeout=300)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    res = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "0 failures" in res.stdout
