"""The C-ABI library loads and exports every call include/zr.h declares, and
the host-side validation of kernel calls rejects bad arguments without a GPU
(no compute call is made here)."""

import ctypes
import os
import re
import shutil
import subprocess

import pytest

from tests._lib import ROOT, LIB, load

zr = load()
HEADER = os.path.join(ROOT, "include", "zr.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(zr_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = _declared()
    for required in ("zr_plan_buckets", "zr_ipg_accumulate",
                     "zr_reduce_scatter_local", "zr_adam_partition",
                     "zr_reduce_scatter_adam", "zr_copy_grads_in_partition",
                     "zr_ring_rs_step", "zr_last_error", "zr_version"):
        assert required in names


def test_every_declared_symbol_is_exported():
    out = subprocess.run(["nm", "-D", "--defined-only", LIB],
                         stdout=subprocess.PIPE, text=True, check=True).stdout
    exported = set(re.findall(r"\s[TW]\s+(\S+)$", out, flags=re.M))
    missing = [n for n in _declared() if n not in exported]
    assert not missing, missing
    lib = ctypes.CDLL(LIB)
    for n in _declared():
        assert hasattr(lib, n)
    # the binding wraps exactly the declared calls
    assert sorted(zr.EXPORTED) == _declared()


def test_version():
    assert zr.zr_version() == 100


class _FakeTensor:
    """Stands in for a tensor where only an address is needed (host-side
    validation rejects the call before anything touches the GPU)."""

    def __init__(self, addr, numel, dtype="fp32"):
        import torch
        self._addr, self._n = addr, numel
        self.dtype = torch.bfloat16 if dtype == "bf16" else torch.float32

    def data_ptr(self):
        return self._addr

    def numel(self):
        return self._n


def _tiny_plan():
    return zr.zr_plan_buckets([37, 2112, 129], [0, 0, 0], [(4, 1)], 1000)


@pytest.mark.parametrize("kwargs,msg", [
    (dict(group=1), "group"),
    (dict(bucket=3), "bucket"),
    (dict(dst=4), "dst"),
])
def test_reduce_rejects_bad_indices(kwargs, msg):
    plan = _tiny_plan()
    reps = [_FakeTensor(0x1000 * (i + 1), 2280) for i in range(4)]
    args = dict(group=0, bucket=-1, dst=-1)
    args.update(kwargs)
    with pytest.raises(zr.ZrError) as ei:
        zr.zr_reduce_scatter_local(plan, args["group"], args["bucket"],
                                   args["dst"], reps,
                                   [_FakeTensor(0x100000, 570)] * 4, stream=0)
    assert ei.value.status == zr.ZR_ERR_INVALID and msg in str(ei.value)


def test_reduce_rejects_window_that_misses_a_slice():
    plan = _tiny_plan()
    # replica 2's window starts one element too late for partition 1
    reps = [(_FakeTensor(0x1000 * (i + 1), 570), 570 + (i == 2)) for i in range(4)]
    with pytest.raises(zr.ZrError) as ei:
        zr.zr_reduce_scatter_local(plan, 0, -1, 1, reps, [_FakeTensor(0x100000, 570)], stream=0)
    assert ei.value.status == zr.ZR_ERR_INVALID and "window" in str(ei.value)


def test_reduce_rejects_misaligned_and_null():
    plan = _tiny_plan()
    reps = [_FakeTensor(0x1000 * (i + 1), 2280) for i in range(4)]
    reps[1] = _FakeTensor(0x2002, 2280)       # fp32 replica not 4-byte aligned
    with pytest.raises(zr.ZrError):
        zr.zr_reduce_scatter_local(plan, 0, -1, -1, reps, [_FakeTensor(0x100000, 570)] * 4, stream=0)
    reps[1] = _FakeTensor(0, 2280)
    with pytest.raises(zr.ZrError):
        zr.zr_reduce_scatter_local(plan, 0, -1, -1, reps, [_FakeTensor(0x100000, 570)] * 4, stream=0)


def test_fused_checks_dst_state_sizes_and_adam():
    plan = _tiny_plan()
    reps = [_FakeTensor(0x1000 * (i + 1), 2280) for i in range(4)]
    buf = _FakeTensor(0x100000, 570)
    # dst = -1 updates every partition: the state spans L = 2280 elements
    with pytest.raises(zr.ZrError, match="touches 2280"):
        zr.zr_reduce_scatter_adam(plan, 0, -1, -1, reps, buf, buf, buf, stream=0)
    with pytest.raises(zr.ZrError, match="dst"):
        zr.zr_reduce_scatter_adam(plan, 0, -1, 4, reps, buf, buf, buf, stream=0)
    with pytest.raises(zr.ZrError, match="step"):
        zr.zr_reduce_scatter_adam(plan, 0, -1, 0, reps, buf, buf, buf, step=0, stream=0)
    with pytest.raises(zr.ZrError, match="betas"):
        zr.zr_reduce_scatter_adam(plan, 0, -1, 0, reps, buf, buf, buf, beta1=1.0, stream=0)


def test_capped_fused_checks_the_cap_then_the_fused_arguments():
    plan = _tiny_plan()
    reps = [_FakeTensor(0x1000 * (i + 1), 2280) for i in range(4)]
    buf = _FakeTensor(0x100000, 570)
    for cap in (0, -3):
        with pytest.raises(zr.ZrError, match="max_workgroups") as ei:
            zr.zr_reduce_scatter_adam_capped(plan, 0, -1, 0, reps, buf, buf, buf,
                                             max_workgroups=cap, stream=0)
        assert ei.value.status == zr.ZR_ERR_INVALID
    with pytest.raises(zr.ZrError, match="dst"):
        zr.zr_reduce_scatter_adam_capped(plan, 0, -1, 4, reps, buf, buf, buf,
                                         max_workgroups=8, stream=0)
    with pytest.raises(zr.ZrError, match="step"):
        zr.zr_reduce_scatter_adam_capped(plan, 0, -1, 0, reps, buf, buf, buf, step=0,
                                         max_workgroups=8, stream=0)


def test_binding_rejects_integers_ctypes_would_wrap():
    """ctypes passes 2**32 + 5 to an int32_t as 5; the binding refuses it
    instead of selecting another partition or bucket."""
    plan = _tiny_plan()
    reps = [_FakeTensor(0x1000 * (i + 1), 2280) for i in range(4)]
    buf = _FakeTensor(0x100000, 570)
    for kwargs, name in ((dict(dst=2 ** 32), "dst"), (dict(group=-(2 ** 31) - 1), "group"),
                         (dict(bucket=2 ** 63), "bucket"), (dict(step=2 ** 64 + 1), "step")):
        args = dict(group=0, bucket=-1, dst=0, step=1)
        args.update(kwargs)
        with pytest.raises(zr.ZrError, match=name) as ei:
            zr.zr_reduce_scatter_adam(plan, args["group"], args["bucket"], args["dst"], reps,
                                      buf, buf, buf, step=args["step"], stream=0)
        assert ei.value.status == zr.ZR_ERR_INVALID
    with pytest.raises(zr.ZrError, match="max_workgroups"):
        zr.zr_reduce_scatter_adam_capped(plan, 0, -1, 0, reps, buf, buf, buf,
                                         max_workgroups=2 ** 32 + 5, stream=0)
    with pytest.raises(zr.ZrError, match="numels"):
        zr.zr_plan_buckets([2 ** 63], [0], [(4, 1)], 1000)
    with pytest.raises(zr.ZrError, match="integer"):
        zr.zr_plan_grad_start_offset(plan, 1, 1.5)
    # integral floats keep working (bucket sizes are often written 5e8)
    assert zr.zr_plan_num_buckets(zr.zr_plan_buckets([10, 20], [0, 0], [(2, 1)], 1e1)) == 3


def test_prepared_call_checks_its_arguments_once():
    plan = _tiny_plan()
    reps = [_FakeTensor(0x1000 * (i + 1), 2280) for i in range(4)]
    buf = _FakeTensor(0x100000, 570)
    with pytest.raises(zr.ZrError, match="max_workgroups"):
        zr.prepare_reduce_scatter_adam(plan, 0, 0, reps, buf, buf, buf, max_workgroups=-1)
    with pytest.raises(zr.ZrError, match="group"):
        zr.prepare_reduce_scatter_adam(plan, 1, 0, reps, buf, buf, buf)
    with pytest.raises(zr.ZrError, match="touches 2280"):
        zr.prepare_reduce_scatter_adam(plan, 0, -1, reps, buf, buf, buf)
    call = zr.prepare_reduce_scatter_adam(plan, 0, 4, reps, buf, buf, buf)
    # the C library still validates every call (nothing reaches a GPU here)
    with pytest.raises(zr.ZrError, match="dst"):
        call(-1, 1, stream=0)
    with pytest.raises(zr.ZrError, match="step"):
        zr.prepare_reduce_scatter_adam(plan, 0, 0, reps, buf, buf, buf)(-1, 0, stream=0)


@pytest.mark.parametrize("first", [False, True])
def test_ipg_rejects_mixed_groups_duplicates_and_overrun(first):
    ipg = zr.zr_ipg_accumulate_first if first else zr.zr_ipg_accumulate
    plan = zr.zr_plan_buckets([10, 20, 30], [0, 1, 0], [(2, 1), (2, 1)], 16)
    g = _FakeTensor(0x1000, 10, "bf16")
    g20 = _FakeTensor(0x2000, 20, "bf16")
    mg = _FakeTensor(0x100000, 40)
    with pytest.raises(zr.ZrError, match="share a group"):
        ipg(plan, [0, 1], [g, g20], mg, stream=0)
    with pytest.raises(zr.ZrError, match="twice"):
        ipg(plan, [0, 0], [g, g], mg, stream=0)
    with pytest.raises(zr.ZrError, match="past"):
        ipg(plan, [0], [g], mg, window_base=1, window_len=40, stream=0)


def test_ipg_rejects_gradient_smaller_than_its_param():
    """A gradient tensor must hold its parameter's elements: the kernel would
    otherwise read past it."""
    plan = _tiny_plan()
    mg = _FakeTensor(0x100000, 2280)
    with pytest.raises(zr.ZrError, match=r"grads\[1\] holds 2111 elements; the call touches 2112"):
        zr.zr_ipg_accumulate(plan, [0, 1], [_FakeTensor(0x1000, 37, "bf16"),
                                            _FakeTensor(0x2000, 2111, "bf16")], mg, stream=0)
    with pytest.raises(zr.ZrError, match="holds 1 elements"):
        zr.zr_ipg_accumulate(plan, [2], [_FakeTensor(0x1000, 1, "bf16")], mg, stream=0)


def test_binding_checks_list_lengths_against_the_group():
    """The C calls index the replica, output and partition arrays by rank, so a
    list of the wrong length is refused before the call."""
    plan = _tiny_plan()                       # one group of 4 replicas
    reps = [_FakeTensor(0x1000 * (i + 1), 2280) for i in range(4)]
    buf = _FakeTensor(0x100000, 570)
    whole = _FakeTensor(0x200000, 2280)
    for short in (reps[:2], reps + reps[:1]):
        with pytest.raises(zr.ZrError, match="reps has"):
            zr.zr_reduce_scatter_local(plan, 0, -1, 0, short, [buf], stream=0)
        with pytest.raises(zr.ZrError, match="reps has"):
            zr.zr_reduce_scatter_adam(plan, 0, -1, 0, short, buf, buf, buf, stream=0)
        with pytest.raises(zr.ZrError, match="reps has"):
            zr.zr_reduce_scatter_adam_capped(plan, 0, -1, 0, short, buf, buf, buf,
                                             max_workgroups=4, stream=0)
        with pytest.raises(zr.ZrError, match="reps has"):
            zr.prepare_reduce_scatter_adam(plan, 0, 0, short, buf, buf, buf)
    with pytest.raises(zr.ZrError, match="part_out has 3 entries; the call needs 4"):
        zr.zr_reduce_scatter_local(plan, 0, -1, -1, reps, [buf] * 3, stream=0)
    with pytest.raises(zr.ZrError, match="part_out has 2 entries; the call needs 1"):
        zr.zr_reduce_scatter_local(plan, 0, -1, 1, reps, [buf] * 2, stream=0)
    with pytest.raises(zr.ZrError, match="parts has 3 entries"):
        zr.zr_all_gather_params(plan, 0, [buf] * 3, whole, stream=0)


def test_noalloc_rejects_tables_beyond_its_array():
    """The no-allocation call stages at most 6,552 segments: a selection with
    more is refused before anything touches a GPU."""
    plan = zr.zr_plan_buckets([1] * 7000, [0] * 7000, [(1, 1)], 1)   # 7000 one-element slices
    reps = [_FakeTensor(0x1000, 7000)]
    buf = _FakeTensor(0x100000, 7000)
    with pytest.raises(zr.ZrError, match="7000 segments; the no-allocation call stages at most 6552") as ei:
        zr.zr_reduce_scatter_adam_noalloc(plan, 0, -1, -1, reps, buf, buf, buf, stream=0)
    assert ei.value.status == zr.ZR_ERR_INVALID


def test_ring_rejects_bad_step_and_overlap():
    bufs = [_FakeTensor(0x100000 * (i + 1), 8 * 16) for i in range(8)]
    with pytest.raises(zr.ZrError, match="step"):
        zr.zr_ring_rs_step(bufs, 16, 7, stream=0)
    over = [_FakeTensor(0x100000, 64), _FakeTensor(0x100000 + 64, 64)]
    with pytest.raises(zr.ZrError, match="overlap"):
        zr.zr_ring_rs_step(over, 32, 0, stream=0)


def test_copy_needs_single_bucket():
    plan = _tiny_plan()
    buf = _FakeTensor(0x100000, 1000)
    with pytest.raises(zr.ZrError, match="bucket"):
        zr.zr_copy_grads_in_partition(plan, 0, -1, 0, buf, buf, stream=0)


def test_adam_rejects_negative_n():
    buf = _FakeTensor(0x100000, 16)
    with pytest.raises(zr.ZrError, match="n must"):
        zr.zr_adam_partition(buf, buf, buf, buf, n=-1, stream=0)


def _c_client(tmp_path, name):
    """Compiles tests/native/<name>.c as C11 against include/zr.h and libzr."""
    exe = str(tmp_path / name)
    libdir = os.path.dirname(LIB)
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-x", "c",
                    "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                    "-I", "/opt/rocm/include",
                    os.path.join(ROOT, "tests", "native", name + ".c"),
                    "-x", "none", "-L", libdir, "-lzr", "-Wl,-rpath," + libdir, "-o", exe],
                   check=True)
    return exe


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_plain_c_client_reproduces_the_golden_plan(tmp_path):
    """include/zr.h compiles as C11 and a C program linked to libzr alone
    reproduces the hand-derived tiny plan through the C ABI."""
    exe = _c_client(tmp_path, "plan_dump")
    out = subprocess.run([exe], stdout=subprocess.PIPE, text=True, check=True).stdout
    golden = os.path.join(ROOT, "tests", "golden", "tiny_plan.txt")
    want = [ln.strip() for ln in open(golden) if ln.strip() and not ln.startswith("#")]
    assert out.strip().splitlines() == want


def test_binding_checks_buffer_types_and_sizes():
    """What an address cannot carry is checked by the binding before the C
    call: element type and the number of elements the call touches."""
    plan = _tiny_plan()
    P = zr.zr_plan_group_info(plan, 0)[2]
    reps = [_FakeTensor(0x100000 * (i + 1), 2278) for i in range(4)]
    ok = _FakeTensor(0x900000, P)
    short = _FakeTensor(0xA00000, P - 1)
    with pytest.raises(zr.ZrError, match="master holds"):
        zr.zr_reduce_scatter_adam(plan, 0, -1, 0, reps, short, ok, ok, stream=0)
    with pytest.raises(zr.ZrError, match="param_bf16 must be bf16"):
        zr.zr_reduce_scatter_adam(plan, 0, -1, 0, reps, ok, ok, ok, ok, stream=0)
    with pytest.raises(zr.ZrError, match="part_out"):
        zr.zr_reduce_scatter_local(plan, 0, -1, 0, reps, [short], stream=0)
    with pytest.raises(zr.ZrError, match="replica 1 must be fp32"):
        zr.zr_reduce_scatter_local(plan, 0, -1, 0,
                                   [reps[0], _FakeTensor(0x200000, 2278, "bf16")] + reps[2:],
                                   [ok], stream=0)
    with pytest.raises(zr.ZrError, match="v holds"):
        zr.zr_adam_partition(ok, ok, ok, short, n=P, stream=0)
    with pytest.raises(zr.ZrError, match="rank_bufs"):
        zr.zr_ring_rs_step([_FakeTensor(0x100000 * (i + 1), 63) for i in range(8)], 8, 0,
                           stream=0)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_plain_c_client_sees_documented_errors(tmp_path):
    """From C: invalid plans and kernel calls return ZR_ERR_INVALID with a
    message in zr_last_error(), before anything is enqueued."""
    exe = _c_client(tmp_path, "abi_errors")
    proc = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert proc.returncode == 0, proc.stdout
    assert proc.stdout.strip().endswith("all ok")


def test_kernel_fingerprints_cover_the_measured_kernels():
    """The build writes one fingerprint per kernel of the code object, keyed
    by the demangled name rocprofv3 reports; every kernel a counter entry in
    profiles/traffic.json was measured on is still there under that name (a
    rename would silently turn the bench's traffic figure to null)."""
    import json
    from zero_partition_aware_amd.build import kernel_hashes
    hashes = kernel_hashes()
    assert len(hashes) >= 50
    assert all(len(h) == 16 for h in hashes.values())
    traffic = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    for key, entry in traffic.items():
        for name in entry["kernel_sha"]:
            assert name in hashes, f"{key}: kernel {name!r} is not in the built library"


def test_range_calls_check_their_range():
    """A bucket range must lie inside the plan; an empty range enqueues
    nothing (and needs no GPU)."""
    plan = _tiny_plan()                      # 3 buckets
    reps = [_FakeTensor(0x1000 * (i + 1), 2280) for i in range(4)]
    buf = _FakeTensor(0x100000, 570)
    for first, count in ((-1, 1), (0, -1), (2, 2), (4, 0)):
        with pytest.raises(zr.ZrError, match="bucket") as ei:
            zr.zr_reduce_scatter_local_range(plan, 0, first, count, 0, reps, [buf], stream=0)
        assert ei.value.status == zr.ZR_ERR_INVALID
        with pytest.raises(zr.ZrError, match="bucket"):
            zr.zr_reduce_scatter_adam_range(plan, 0, first, count, 0, reps, buf, buf, buf,
                                            stream=0)
    for first in (0, 3):
        zr.zr_reduce_scatter_local_range(plan, 0, first, 0, 0, reps, [buf], stream=0)
        zr.zr_reduce_scatter_adam_range(plan, 0, first, 0, 1, reps, buf, buf, buf, stream=0)
    call = zr.prepare_reduce_scatter_adam(plan, 0, 2, reps, buf, buf, buf)
    call(1, 1, stream=0, count=0)
    with pytest.raises(zr.ZrError, match="bucket"):
        call(1, 1, stream=0, count=3)


def test_binding_handles_a_group_without_params():
    """A group that no param belongs to has no elements (P_g = 0); list
    lengths are still checked against its world size."""
    plan = zr.zr_plan_buckets([10, 20], [0, 0], [(2, 1), (4, 1)], 16)
    assert zr.zr_plan_group_info(plan, 1)[:3] == (0, 0, 0)
    reps = [_FakeTensor(0x1000 * (i + 1), 30) for i in range(4)]
    zr.zr_reduce_scatter_local(plan, 1, -1, 0, reps, [_FakeTensor(0x100000, 0)], stream=0)
    with pytest.raises(zr.ZrError, match="reps has 3 entries; the call needs 4"):
        zr.zr_reduce_scatter_local(plan, 1, -1, 0, reps[:3], [_FakeTensor(0x100000, 0)], stream=0)


def test_reduce_launch_shape_follows_the_stated_rules():
    """zr_plan_reduce_launches against the launch rules the header states,
    worked out from the oracle plan: a tile is 512 elements for the bf16
    fused step and 256 otherwise, a segment of n elements spans
    (n + 63 + tile - 1) // tile tiles (padding included), and a selection is
    cut into ceil(tiles / floor(2^31 / tile bytes)) equal launches."""
    from oracle.plan import plan_oracle

    def rule(ref, g, first, last, dst, bf16, fused, gout):
        info = ref.groups[g]
        tile = 512 if bf16 and fused else 256
        segs = [s.numel for s in ref.slices
                if s.group == g and first <= s.bucket < last and (dst < 0 or s.dst == dst)]
        if last == ref.num_buckets:
            for d in ([dst] if dst >= 0 else range(info.world)):
                pad = max(0, min(info.part_numel, (d + 1) * info.part_numel - info.total))
                if pad:
                    segs.append(pad)
        tiles = sum((n + 63 + tile - 1) // tile for n in segs)
        tb = tile * (info.world * (2 if bf16 else 4) + ((26 + (4 if gout else 0)) if fused else 4))
        per = (2 ** 31) // tb
        return tiles, (-(-tiles // per) if tiles else 0)

    cases = [([37, 64 * 33, 129], [0, 0, 0], [(4, 1)], 1000),
             ([8 * 40_000_000 - 10], [0], [(8, 1)], 290_000_000),
             ([36_000_000], [0], [(4, 1)], 13_500_000),
             ([300_000, 5, 70_000, 1_234_567], [0, 1, 0, 1], [(8, 2), (2, 2)], 100_000)]
    for numels, pg, groups, B in cases:
        ref = plan_oracle(numels, pg, groups, B)
        plan = zr.zr_plan_buckets(numels, pg, groups, B)
        nb = ref.num_buckets
        for g in range(len(groups)):
            for dst in [-1] + list(range(groups[g][0])):
                for first, last in [(0, nb), (0, 1), (nb - 1, nb), (nb // 2, nb)]:
                    for bf16 in (False, True):
                        for fused, gout in ((False, False), (True, False), (True, True)):
                            got = zr.zr_plan_reduce_launches(
                                plan, g, first, last - first, dst, "bf16" if bf16 else "fp32",
                                fused, gout)
                            assert got == rule(ref, g, first, last, dst, bf16, fused, gout), \
                                (numels, g, dst, first, last, bf16, fused, gout)
    with pytest.raises(zr.ZrError):
        zr.zr_plan_reduce_launches(plan, 0, 0, nb + 1, 0, "fp32", True)
    with pytest.raises(zr.ZrError):
        zr.zr_plan_reduce_launches(plan, 0, 0, 1, 99, "fp32", True)
    with pytest.raises(zr.ZrError):
        zr.zr_plan_reduce_launches(plan, 0, 0, 1, 0, "fp16", True)


def test_reduce_launch_occupancy_follows_the_stated_table():
    """zr_reduce_launch_occupancy against the table the library states: at
    8 replicas fp32 fused 8, bf16 fused 6, bf16 reduce-scatter 20, fp32
    reduce-scatter 12 workgroups per CU; at 4 replicas fp32 fused 14, bf16
    fused 7; at 16 replicas fp32 fused 6, fp32 reduce-scatter 7; at 2
    replicas fp32 fused 18; every other shape 0 (register-limited); the
    XCD-weighted order from 2 replicas up."""
    def rule(bf16, fused, world):
        if world == 8:
            return (6 if bf16 else 8) if fused else (20 if bf16 else 12)
        if world == 4 and fused:
            return 7 if bf16 else 14
        if world == 16 and not bf16:
            return 6 if fused else 7
        if world == 2 and not bf16 and fused:
            return 18
        return 0

    for world in list(range(1, 18)) + [64]:
        for bf16 in (False, True):
            for fused in (False, True):
                got = zr.zr_reduce_launch_occupancy("bf16" if bf16 else "fp32", fused, world)
                assert got == (rule(bf16, fused, world), world >= 2), (world, bf16, fused)
    for bad in ((0, "fp32"), (-3, "bf16"), (8, "fp16")):
        with pytest.raises(zr.ZrError):
            zr.zr_reduce_launch_occupancy(bad[1], True, bad[0])
