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


# Per-kernel fingerprints of the device code: for every kernel in the gfx950
# code object, a hash of its instruction bytes (.text) and of its kernel
# descriptor (.rodata, register and segment sizes), written beside the
# library at build time as {demangled kernel name: hash}.  The code holds no
# relocations or PC-relative references, so a kernel's bytes do not depend on
# where it sits; the descriptor's code-entry offset, which does, is zeroed
# before hashing.  A counter measurement stays tied to exactly the kernel it
# was taken on: host-side edits, or changes to other kernels, leave it valid.
KERNEL_SHA = os.path.join(HERE, "libzr.kernels.json")
_KD_ENTRY_OFFSET = slice(16, 24)   # kernel_code_entry_byte_offset in a descriptor


def _llvm_tool(name):
    for cand in (f"/opt/rocm/llvm/bin/{name}", shutil.which(name)):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError(f"{name} not found: the ROCm LLVM tools are required")


def _kernel_hashes(hipcc):
    import hashlib
    import json
    import tempfile
    with tempfile.TemporaryDirectory() as tmp:
        obj = os.path.join(tmp, "dev.o")
        _run([hipcc, *HIP_FLAGS, "-I", INCLUDE, "-I", CSRC, "--cuda-device-only",
              "--no-gpu-bundle-output", "-c", os.path.join(CSRC, "zr_kernels.hip"),
              "-o", obj])
        readelf = _llvm_tool("llvm-readelf")
        sections = {}
        for ln in _run([readelf, "-S", "--wide", obj]).splitlines():
            f = ln.replace("[ ", "[").split()
            if len(f) > 5 and f[1] in (".text", ".rodata"):
                sections[f[1]] = (int(f[3], 16), int(f[4], 16))   # address, file offset
        funcs, descs = {}, {}
        for ln in _run([readelf, "-s", "--wide", obj]).splitlines():
            f = ln.split()
            if len(f) == 8 and f[3] in ("FUNC", "OBJECT"):
                addr, size, name = int(f[1], 16), int(f[2]), f[7]
                if f[3] == "FUNC":
                    funcs[name] = (addr, size)
                elif name.endswith(".kd"):
                    descs[name[:-3]] = (addr, size)
        with open(obj, "rb") as fh:
            data = fh.read()

        def read(sec, addr, size):
            base, off = sections[sec]
            return data[off + addr - base: off + addr - base + size]

        names = sorted(funcs)
        demangled = _run(["c++filt"] + names).splitlines() if names else []
        out = {}
        for name, dname in zip(names, demangled):
            if name not in descs:
                continue
            kd = bytearray(read(".rodata", *descs[name]))
            kd[_KD_ENTRY_OFFSET] = bytes(_KD_ENTRY_OFFSET.stop - _KD_ENTRY_OFFSET.start)
            h = hashlib.sha256(read(".text", *funcs[name]) + bytes(kd))
            out[dname.strip()] = h.hexdigest()[:16]
        if not out:
            raise RuntimeError("no kernels found in the device code object")
        return json.dumps(out, indent=1, sort_keys=True) + "\n"


def kernel_hashes():
    """{demangled kernel name: fingerprint} of the built library's kernels
    (empty if not built)."""
    import json
    try:
        with open(KERNEL_SHA) as fh:
            return json.load(fh)
    except (OSError, ValueError):
        return {}


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
    # The fingerprints only gate counter figures in bench.py: without them
    # (tools missing) the library is still built and `traffic` reads null.
    try:
        text = _kernel_hashes(hipcc)
    except (RuntimeError, OSError) as e:
        if os.path.exists(KERNEL_SHA):
            os.remove(KERNEL_SHA)
        print(f"warning: kernel fingerprints not written ({e})", file=sys.stderr)
    else:
        with open(KERNEL_SHA, "w") as fh:
            fh.write(text)
    if verbose:
        print(out)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
