"""Compile libzr.so (host planner + HIP kernels for gfx950) in-tree.

Run as ``python -m zero_partition_aware_amd.build``; ``__graft_entry__.build``
calls ``build()``.  Every call recompiles.
"""

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libzr.so")
ARCH = os.environ.get("ZR_OFFLOAD_ARCH", "gfx950")


def _hipcc():
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required")


# Flags shared by every HIP compile: no FMA contraction (the reduction must
# round exactly as its definition), IEEE denormals kept (the default), and
# no packed-fp32 instructions.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-ffp-contract=off", "-fno-fast-math",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _code_text(path):
    """A C/C++ source with its comments removed and whitespace collapsed: the
    part of the file that reaches the compiler."""
    import re
    with open(path) as fh:
        text = fh.read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_hash():
    """Short hash of the device code and its compile flags (comments and
    whitespace excluded): counter measurements are only valid for the exact
    code they were taken on."""
    import hashlib
    h = hashlib.sha256()
    for path in (os.path.join(CSRC, "zr_kernels.hip"), os.path.join(CSRC, "zr_internal.h"),
                 os.path.join(INCLUDE, "zr.h")):
        h.update(_code_text(path).encode())
    h.update(" ".join(HIP_FLAGS).encode())
    return h.hexdigest()[:16]


def _run(cmd):
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                          text=True)
    if proc.returncode != 0:
        raise RuntimeError("build step failed:\n" + " ".join(cmd) + "\n" +
                           proc.stdout)
    return proc.stdout


def build(verbose=False):
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    plan_o = os.path.join(BUILD_DIR, "zr_plan.o")
    kern_o = os.path.join(BUILD_DIR, "zr_kernels.o")
    # The planner is plain C++ (no device code): compiled by the host compiler.
    out = _run(["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra",
                "-D__HIP_PLATFORM_AMD__", "-I", INCLUDE, "-I", CSRC,
                "-I", "/opt/rocm/include", "-c",
                os.path.join(CSRC, "zr_plan.cpp"), "-o", plan_o])
    out += _run([hipcc, *HIP_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c",
                 os.path.join(CSRC, "zr_kernels.hip"), "-o", kern_o])
    tmp = LIB + ".tmp"
    # The HIP runtime is a dependency by soname (libamdhip64.so.7): in a
    # process that already holds torch's copy of the runtime (same soname) the
    # loader reuses it; standalone, RUNPATH finds the ROCm installation's.
    out += _run(["g++", "-shared", "-fPIC", plan_o, kern_o,
                 "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib",
                 "-Wl,--no-undefined", "-o", tmp])
    os.replace(tmp, LIB)
    if verbose:
        print(out)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
