"""The host planner under AddressSanitizer + UndefinedBehaviorSanitizer.

Builds tests/native/planner_fuzz.cpp with the planner source (plain C++, no
device code) using g++ and runs it on random plans; any memory error or
undefined behaviour aborts the run."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_planner_fuzz_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "planner_fuzz")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "zero_partition_aware_amd", "csrc"),
           "-I", "/opt/rocm/include",
           os.path.join(ROOT, "tests", "native", "planner_fuzz.cpp"),
           os.path.join(ROOT, "zero_partition_aware_amd", "csrc", "zr_plan.cpp"),
           "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    out = subprocess.run([exe, "300"], capture_output=True, text=True, env=env, timeout=300)
    assert out.returncode == 0, out.stdout + out.stderr
    assert "planner fuzz ok" in out.stdout
