"""Every kernel of the library run on the CPU under AddressSanitizer +
UndefinedBehaviorSanitizer: the library's own sources (zr_kernels.hip compiled
as C++ against tests/native/emu, the planner) driven through the C ABI by
tests/native/kernel_emu.cpp on random plans, selections, element types,
windows and pointer offsets, with tiny launch caps so that small cases take
the multi-launch path, and a short XCD-weighted tile cycle so that they take
its idle slots too.  Any access
outside a buffer (vector accesses to the byte, scalar ones at ASan's
granularity), any store before a buffer, and any output that differs from a
plain loop over the plan's slices fails the run.  The coverage report must
name every kernel variant, and a planted one-slot shift of a store base must
be caught."""

import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang++"
CSRC = os.path.join(ROOT, "zero_partition_aware_amd", "csrc")
NATIVE = os.path.join(ROOT, "tests", "native")

pytestmark = pytest.mark.skipif(not os.path.exists(CLANG), reason="ROCm clang++ not available")

ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1:verify_asan_link_order=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _build(tmp_path, kernels_src, name):
    exe = str(tmp_path / name)
    cmd = [CLANG, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-ffp-contract=off",
           "-Wno-align-mismatch", "-D__HIP_PLATFORM_AMD__", "-DZR_LAUNCH_BYTES=65536",
           # an XCD-weighted order of 2-round cycles (from 2 replicas up, as
           # in the library), so that short launches hold whole cycles; one
           # replica and capped calls keep equal shares
           "-DZR_XCD_SKEW=2",
           "-I", os.path.join(NATIVE, "emu"), "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-I", "/opt/rocm/include",
           "-x", "c++", kernels_src, "-x", "none", os.path.join(CSRC, "zr_plan.cpp"),
           os.path.join(NATIVE, "emu", "emu_runtime.cpp"), os.path.join(NATIVE, "kernel_emu.cpp"),
           "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return exe


# Every kernel and variant the random cases must reach (name prefixes as the
# coverage report prints them).
REQUIRED = [
    # fused, common / dword-aligned, bf16 and fp32, 8 replicas
    "reduce_kernel<float, 8, false, true, false>",
    "reduce_kernel<float, 8, false, true, true>",
    "reduce_kernel<unsigned short, 8, false, true, false>",
    "reduce_kernel<unsigned short, 8, false, true, true>",
    # unfused, run-time replica count, true division
    "reduce_kernel<float, 8, false, false, false>",
    "reduce_kernel<unsigned short, 0, ",
    "reduce_kernel<float, 3, true, ",
    "adam_kernel<true, false>", "adam_kernel<true, true>", "adam_kernel<false, false>",
    "ipg_kernel<float, false, false>", "ipg_kernel<float, true, false>",
    "ipg_kernel<unsigned short, false, false>", "ipg_kernel<unsigned short, true, false>",
    "ipg_kernel<float, false, true>", "ipg_kernel<float, true, true>",
    "ipg_kernel<unsigned short, false, true>", "ipg_kernel<unsigned short, true, true>",
    "copy_kernel<false>", "copy_kernel<true>",
    "gather_kernel<float, false>", "gather_kernel<float, true>",
    "gather_kernel<unsigned short, false>", "gather_kernel<unsigned short, true>",
    "ring_kernel<false>", "ring_kernel<true>", "ring_ag_kernel<false>", "ring_ag_kernel<true>",
    "stage_segs_kernel",
]


def test_every_kernel_on_cpu_under_asan_ubsan(tmp_path):
    exe = _build(tmp_path, os.path.join(CSRC, "zr_kernels.hip"), "kernel_emu")
    out = subprocess.run([exe, "6000"], capture_output=True, text=True, env=ENV, timeout=600)
    assert out.returncode == 0, out.stdout[-3000:] + out.stderr[-3000:]
    assert "kernel emulation ok: 6000 cases" in out.stdout
    cov = {}
    for ln in out.stdout.splitlines():
        m = re.match(r"launches (\d+) (.*)$", ln)
        if m:
            cov[m.group(2)] = int(m.group(1))
    for name in REQUIRED:
        assert any(k.startswith(name) and n > 0 for k, n in cov.items()), \
            f"no launch of {name}: {sorted(cov)}"


def test_planted_store_shift_is_caught(tmp_path):
    """A copy of the kernel source whose fused Adam writes the master one
    4-element slot late (in a temporary file, never in the library) must
    fail the check."""
    src = open(os.path.join(CSRC, "zr_kernels.hip")).read()
    line = "      b_master = reinterpret_cast<uint64_t>(a.master) + p4;"
    assert src.count(line) == 1
    mutant = tmp_path / "zr_kernels_mutant.hip"
    mutant.write_text(src.replace(line, line[:-1] + " + 16;"))
    exe = _build(tmp_path, str(mutant), "kernel_emu_mutant")
    out = subprocess.run([exe, "200"], capture_output=True, text=True, env=ENV, timeout=600)
    assert out.returncode != 0
    assert "out-of-bounds" in out.stderr or "FAIL" in out.stderr
