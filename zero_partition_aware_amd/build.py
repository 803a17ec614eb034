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


# The device code's fingerprint: a hash of the gfx950 code object's
# instructions (.text), kernel descriptors (.rodata) and kernel metadata
# (.note), written beside the library at build time.  The rest of the ELF
# (build ids, symbol tables) differs from compile to compile, and host-side
# edits leave these sections alone, so counter measurements stay tied to the
# exact kernels they were taken on.
DEVICE_SHA = os.path.join(HERE, "libzr.device_sha")
DEVICE_SECTIONS = (".text", ".rodata", ".note")


def _objcopy():
    for cand in ("/opt/rocm/llvm/bin/llvm-objcopy", shutil.which("llvm-objcopy")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("llvm-objcopy not found: the ROCm LLVM tools are required")


def _device_code_hash(hipcc):
    import hashlib
    import tempfile
    with tempfile.TemporaryDirectory() as tmp:
        obj = os.path.join(tmp, "dev.o")
        _run([hipcc, *HIP_FLAGS, "-I", INCLUDE, "-I", CSRC, "--cuda-device-only",
              "--no-gpu-bundle-output", "-c", os.path.join(CSRC, "zr_kernels.hip"),
              "-o", obj])
        h = hashlib.sha256()
        for sec in DEVICE_SECTIONS:
            out = os.path.join(tmp, "sec.bin")
            _run([_objcopy(), "--dump-section", f"{sec}={out}", obj])
            with open(out, "rb") as fh:
                data = fh.read()
            h.update(sec.encode() + len(data).to_bytes(8, "little") + data)
        return h.hexdigest()[:16]


def device_code_hash():
    """Fingerprint of the built library's device code (None if not built)."""
    try:
        with open(DEVICE_SHA) as fh:
            return fh.read().strip() or None
    except OSError:
        return None


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
    with open(DEVICE_SHA, "w") as fh:
        fh.write(_device_code_hash(hipcc) + "\n")
    if verbose:
        print(out)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
