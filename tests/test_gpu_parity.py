"""HIP path vs the oracle, element by element, at sizes the oracle finishes in
seconds: many tiles, ragged tails, misaligned pointers,
several groups, power-of-two and other divisors, special values."""

import random

import numpy as np
import pytest

from oracle.adam import adam_oracle
from oracle.bf16 import bf16_rne_oracle
from oracle.copy import bucket_layout_mean, copy_grads_in_partition_oracle
from oracle.ipg import ipg_accumulate_oracle
from oracle.plan import plan_oracle
from oracle.reduce import reduce_scatter_oracle
from oracle.ring import ring_reduce_scatter_oracle, ring_order_sum
from tests._lib import load
from zero_partition_aware_amd import workloads

pytestmark = pytest.mark.gpu

zr = load()
torch = pytest.importorskip("torch")
from tests._gpu import (assert_bits_equal, assert_within, empty_f32,  # noqa: E402
                        host_f32, host_u16, max_ulp, to_dev)

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8)


def _draw(rng, n, is_bf16, sigma=1.0, special=False):
    if special:
        x = workloads.host_special_values(rng.integers(1 << 30), n)
    else:
        x = (rng.standard_normal(n) * sigma).astype(np.float32)
    if is_bf16:
        return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return x


def _make_case(seed):
    rng = random.Random(seed)
    ng = rng.choice([1, 1, 2])
    groups = []
    for _ in range(ng):
        R = rng.choice([1, 2, 3, 4, 5, 6, 8, 8, 12, 16])
        sp = rng.choice([d for d in (1, 2, 3, 4) if R % d == 0])
        groups.append((R, sp))
    n = rng.randint(1, 12)
    numels = [rng.choice([1, 3, 17, rng.randint(1, 30000)]) for _ in range(n)]
    pg = [rng.randrange(ng) for _ in range(n)]
    B = rng.choice([1000, 4096, 7777, 30000, 1 << 30])
    align = rng.choice([1, 1, 8])
    return numels, pg, groups, B, align


@pytest.mark.parametrize("seed", range(12))
@pytest.mark.parametrize("is_bf16", [False, True])
def test_reduce_scatter_random_plans(seed, is_bf16):
    numels, pg, groups, B, align = _make_case(seed)
    ref = plan_oracle(numels, pg, groups, B, align)
    plan = zr.zr_plan_buckets(numels, pg, groups, B, 0, align)
    rng = np.random.default_rng(seed)
    for g, info in enumerate(ref.groups):
        if info.total == 0:
            continue
        reps = [_draw(rng, info.total, is_bf16) for _ in range(info.world)]
        offs = [0] * info.world if seed % 3 else [r % 3 for r in range(info.world)]
        dreps = [to_dev(x, o) for x, o in zip(reps, offs)]
        want = reduce_scatter_oracle(ref, g, reps, is_bf16)
        outs = [empty_f32(info.part_numel, offset_elems=seed % 2) for _ in range(info.world)]
        zr.zr_reduce_scatter_local(plan, g, -1, -1, dreps, outs)
        for k in range(info.world):
            assert_bits_equal(host_f32(outs[k]), want[k], f"group {g} dst {k}")


@pytest.mark.parametrize("is_bf16", [False, True])
def test_per_bucket_per_dst_calls_compose(is_bf16):
    w = workloads.get("tiny")
    ref = plan_oracle(w.numels, w.param_groups, w.groups, w.reduce_bucket_size)
    plan = zr.zr_plan_buckets(w.numels, w.param_groups, w.groups, w.reduce_bucket_size)
    rng = np.random.default_rng(3)
    reps = [_draw(rng, 2278, is_bf16) for _ in range(4)]
    dreps = [to_dev(x) for x in reps]
    whole = reduce_scatter_oracle(ref, 0, reps, is_bf16)
    for k in range(4):
        out = empty_f32(570)
        for b in range(ref.num_buckets):
            zr.zr_reduce_scatter_local(plan, 0, b, k, dreps, [out])
        assert_bits_equal(host_f32(out), whole[k], f"dst {k}")


def test_tiny_workload_with_windowed_replicas():
    w = workloads.get("tiny")
    ref = plan_oracle(w.numels, w.param_groups, w.groups, w.reduce_bucket_size)
    plan = zr.zr_plan_buckets(w.numels, w.param_groups, w.groups, w.reduce_bucket_size)
    reps = [workloads.host_normal(workloads.seed_for("tiny", r), 2278, 1.0) for r in range(4)]
    whole = reduce_scatter_oracle(ref, 0, reps, False)
    for k in range(4):
        lo, hi = k * 570, min(2278, (k + 1) * 570)
        win = [(to_dev(x[lo:hi]), lo) for x in reps]
        out = empty_f32(570)
        zr.zr_reduce_scatter_local(plan, 0, -1, k, win, [out])
        assert_bits_equal(host_f32(out), whole[k], f"dst {k}")


@pytest.mark.parametrize("R,sp", [(4, 1), (4, 4), (3, 1), (6, 2), (1, 1)])
def test_special_values(R, sp):
    numels = [4096 * 2 + 5, 3, 1000]
    ref = plan_oracle(numels, [0, 0, 0], [(R, sp)], 5000)
    plan = zr.zr_plan_buckets(numels, [0, 0, 0], [(R, sp)], 5000)
    info = ref.groups[0]
    rng = np.random.default_rng(R * 10 + sp)
    reps = [_draw(rng, info.total, False, special=True) for _ in range(R)]
    want = reduce_scatter_oracle(ref, 0, reps, False)
    outs = [empty_f32(info.part_numel) for _ in range(R)]
    with np.errstate(all="ignore"):
        zr.zr_reduce_scatter_local(plan, 0, -1, -1, [to_dev(x) for x in reps], outs)
        for k in range(R):
            assert_bits_equal(host_f32(outs[k]), want[k], f"dst {k}")


def test_subnormal_and_overflow_probes():
    # x/4 of a subnormal must not flush; 4 x 3e38 pre-divided stays finite.
    vals = np.array([2.0 ** -140, 3e38, -3e38, 1e-45, -0.0], np.float32)
    plan = zr.zr_plan_buckets([5], [0], [(4, 1)], 100)
    ref = plan_oracle([5], [0], [(4, 1)], 100)
    reps = [vals.copy() for _ in range(4)]
    outs = [empty_f32(2) for _ in range(4)]
    zr.zr_reduce_scatter_local(plan, 0, -1, -1, [to_dev(x) for x in reps], outs)
    got = np.concatenate([host_f32(o) for o in outs])[:5]
    want = np.concatenate([reduce_scatter_oracle(ref, 0, reps, False)[k] for k in range(4)])[:5]
    assert_bits_equal(got, want)
    assert got[0] == np.float32(2.0 ** -140) and got[1] == np.float32(3e38)
    assert np.signbit(got[4])


@pytest.mark.parametrize("n,off", [(1, 0), (4095, 0), (4096 * 3 + 7, 0), (20011, 1), (20011, 3)])
@pytest.mark.parametrize("step", [1, 2])
def test_adam_partition(n, off, step):
    rng = np.random.default_rng(n + off + step)
    g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    th = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-4).astype(np.float32) if step > 1 else np.zeros(n, np.float32)
    v = (np.abs(rng.standard_normal(n)) * 1e-7).astype(np.float32) if step > 1 else np.zeros(n, np.float32)
    dg, dth, dm, dv = to_dev(g, off), to_dev(th, off), to_dev(m, off), to_dev(v, off)
    pb = torch.zeros(n + off + 8, dtype=torch.bfloat16, device="cuda")[off: off + n]
    zr.zr_adam_partition(dg, dth, dm, dv, pb, step=step, **HP)
    w_th, w_m, w_v = adam_oracle(g, th, m, v, step=step, **HP)
    gth, gm, gv = host_f32(dth), host_f32(dm), host_f32(dv)
    assert_within(gth, w_th, what="master")
    assert_within(gm, w_m, what="m")
    assert_within(gv, w_v, atol=0.0, what="v")
    # bf16 writeback = RNE of the GPU's own fp32 master, bit for bit.
    assert np.array_equal(host_u16(pb), bf16_rne_oracle(gth))
    print(f"adam n={n} step={step}: max ulp master {max_ulp(gth, w_th)}, "
          f"m {max_ulp(gm, w_m)}, v {max_ulp(gv, w_v)}")


# fp32 buffers 1-3 elements off a 16-byte boundary with the bf16 output on an
# even element (or absent): the dword-aligned variant of the Adam kernel.
# Equal to the oracle, and bit for bit to the same call on aligned copies.
@pytest.mark.parametrize("offs", [(1, 2), (2, 0), (3, None), (1, 1)])
def test_adam_partition_dword_offsets(offs):
    off, pb_off = offs
    n = 4096 * 5 + 13
    rng = np.random.default_rng(off)
    g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    th = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    v = (np.abs(rng.standard_normal(n)) * 1e-7).astype(np.float32)
    res = {}
    for how, o, po in (("offset", off, pb_off), ("aligned", 0, 0)):
        dg, dth, dm, dv = to_dev(g, o), to_dev(th, o), to_dev(m, o), to_dev(v, o)
        pb = (None if po is None else
              torch.zeros(n + po + 8, dtype=torch.bfloat16, device="cuda")[po: po + n])
        zr.zr_adam_partition(dg, dth, dm, dv, pb, step=3, **HP)
        res[how] = [host_f32(dth), host_f32(dm), host_f32(dv)] + (
            [] if pb is None else [host_u16(pb)])
    for a_, b_, nm in zip(res["offset"], res["aligned"], ("master", "m", "v", "bf16")):
        assert np.array_equal(a_.view(np.uint8), b_.view(np.uint8)), f"{nm}: offset vs aligned"
    w_th, w_m, w_v = adam_oracle(g, th, m, v, step=3, **HP)
    assert_within(res["offset"][0], w_th, what="master")
    assert_within(res["offset"][1], w_m, what="m")
    assert_within(res["offset"][2], w_v, atol=0.0, what="v")


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("is_bf16", [False, True])
def test_fused_equals_unfused_and_oracle(seed, is_bf16):
    numels, pg, groups, B, align = _make_case(100 + seed)
    ref = plan_oracle(numels, pg, groups, B, align)
    plan = zr.zr_plan_buckets(numels, pg, groups, B, 0, align)
    rng = np.random.default_rng(seed)
    for g, info in enumerate(ref.groups):
        if info.total == 0:
            continue
        P = info.part_numel
        reps = [_draw(rng, info.total, is_bf16, sigma=1e-3) for _ in range(info.world)]
        dreps = [to_dev(x) for x in reps]
        want_g = reduce_scatter_oracle(ref, g, reps, is_bf16)
        for k in sorted({0, info.world - 1}):
            th = (rng.standard_normal(P) * 0.02).astype(np.float32)
            first = max(0, min(P, info.total - k * P))
            th[first:] = 0.0                       # padding holds zeros
            m = np.zeros(P, np.float32)
            v = np.zeros(P, np.float32)
            off = seed % 2
            # fused
            fth, fm, fv = to_dev(th, off), to_dev(m, off), to_dev(v, off)
            fpb = torch.zeros(P + 8, dtype=torch.bfloat16, device="cuda")[:P]
            fgo = empty_f32(P, off)
            zr.zr_reduce_scatter_adam(plan, g, -1, k, dreps, fth, fm, fv, fpb, fgo, **HP)
            # unfused
            ug = empty_f32(P)
            zr.zr_reduce_scatter_local(plan, g, -1, k, dreps, [ug])
            uth, um, uv = to_dev(th), to_dev(m), to_dev(v)
            upb = torch.zeros(P, dtype=torch.bfloat16, device="cuda")
            zr.zr_adam_partition(ug, uth, um, uv, upb, **HP)
            assert_bits_equal(host_f32(fgo), host_f32(ug), "grad fused vs unfused")
            assert_bits_equal(host_f32(fgo), want_g[k], "grad vs oracle")
            for a, b, nm in ((fth, uth, "master"), (fm, um, "m"), (fv, uv, "v")):
                assert_bits_equal(host_f32(a), host_f32(b), nm + " fused vs unfused")
            assert np.array_equal(host_u16(fpb), host_u16(upb))
            w_th, w_m, w_v = adam_oracle(want_g[k], th, m, v, step=1, **HP)
            assert_within(host_f32(fth), w_th, what="master vs oracle")
            assert_within(host_f32(fm), w_m, what="m vs oracle")
            assert_within(host_f32(fv), w_v, atol=0.0, what="v vs oracle")
            assert (host_f32(fth)[first:] == 0).all()


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("is_bf16", [False, True])
@pytest.mark.parametrize("per_bucket", [False, True])
def test_fused_every_partition_in_one_call(seed, is_bf16, per_bucket):
    """dst = -1 with state buffers over the whole padded flat space: one
    launch (or one per bucket) updates every partition; each partition equals
    the oracle and, bit for bit, its own single-partition call."""
    numels, pg, groups, B, align = _make_case(200 + seed)
    ref = plan_oracle(numels, pg, groups, B, align)
    plan = zr.zr_plan_buckets(numels, pg, groups, B, 0, align)
    rng = np.random.default_rng(50 + seed)
    off = seed % 2
    for g, info in enumerate(ref.groups):
        if info.total == 0:
            continue
        P, R, L = info.part_numel, info.world, info.padded
        reps = [_draw(rng, info.total, is_bf16, sigma=1e-3) for _ in range(R)]
        dreps = [to_dev(x) for x in reps]
        want_g = reduce_scatter_oracle(ref, g, reps, is_bf16)
        th = (rng.standard_normal(L) * 0.02).astype(np.float32)
        m = (rng.standard_normal(L) * 1e-4).astype(np.float32)
        v = np.abs(rng.standard_normal(L) * 1e-8).astype(np.float32)
        th[info.total:] = m[info.total:] = v[info.total:] = 0.0
        ath, am, av = to_dev(th, off), to_dev(m, off), to_dev(v, off)
        apb = torch.zeros(L + 8, dtype=torch.bfloat16, device="cuda")[off: off + L]
        ago = empty_f32(L, off)
        for b in (range(ref.num_buckets) if per_bucket else [-1]):
            zr.zr_reduce_scatter_adam(plan, g, b, -1, dreps, ath, am, av, apb, ago, step=2, **HP)
        got = [host_f32(t) for t in (ago, ath, am, av)] + [host_u16(apb)]
        for k in range(R):
            sl = slice(k * P, (k + 1) * P)
            kth, km, kv = to_dev(th[sl]), to_dev(m[sl]), to_dev(v[sl])
            kpb = torch.zeros(P, dtype=torch.bfloat16, device="cuda")
            kgo = empty_f32(P)
            zr.zr_reduce_scatter_adam(plan, g, -1, k, dreps, kth, km, kv, kpb, kgo, step=2, **HP)
            one = [host_f32(t) for t in (kgo, kth, km, kv)] + [host_u16(kpb)]
            for a_, b_, nm in zip(got, one, ("grad", "master", "m", "v", "bf16")):
                assert np.array_equal(a_[sl].view(np.uint8), b_.view(np.uint8)), \
                    f"{nm} of partition {k}: every-partition call vs its own call"
            assert_bits_equal(got[0][sl], want_g[k], f"grad of partition {k} vs oracle")
            w_th, w_m, w_v = adam_oracle(want_g[k], th[sl], m[sl], v[sl], step=2, **HP)
            assert_within(got[1][sl], w_th, what=f"master of partition {k}")
            assert_within(got[2][sl], w_m, what=f"m of partition {k}")
            assert_within(got[3][sl], w_v, atol=0.0, what=f"v of partition {k}")
            assert np.array_equal(got[4][sl], bf16_rne_oracle(got[1][sl]))


# Element offsets of (replicas, master / m / v / reduced-grad outputs, bf16
# param) inside their allocations.  Each nonzero choice gives the first
# segment of some partition a nonzero tile phase (replica tiles moved onto
# whole 128-byte lines, or one slot phase shared by every stream), so that
# segment's first tile starts before partition offset 0 and the per-tile
# stream bases are formed from a negative element offset.
@pytest.mark.parametrize("is_bf16", [True, False])
@pytest.mark.parametrize("offs", [(0, 0, 0), (32, 0, 0), (1, 1, 1), (3, 3, 3),
                                  (33, 1, 1), (17, 0, 0)])
def test_tile_phase_at_partition_start(is_bf16, offs):
    ro, so, po = offs
    numels, R = [12345, 7654], 4                 # 19,999 elements: P = 5000, 1 pad
    ref = plan_oracle(numels, [0, 0], [(R, 1)], 1 << 30)
    plan = zr.zr_plan_buckets(numels, [0, 0], [(R, 1)], 1 << 30)
    P = ref.groups[0].part_numel
    rng = np.random.default_rng(7 * sum(offs) + int(is_bf16))
    reps = [_draw(rng, ref.groups[0].total, is_bf16, sigma=1e-3) for _ in range(R)]
    dreps = [to_dev(x, ro) for x in reps]
    want_g = reduce_scatter_oracle(ref, 0, reps, is_bf16)
    for k in range(R):
        th = (rng.standard_normal(P) * 0.02).astype(np.float32)
        m = (rng.standard_normal(P) * 1e-4).astype(np.float32)
        v = np.abs(rng.standard_normal(P) * 1e-8).astype(np.float32)
        first = max(0, min(P, ref.groups[0].total - k * P))
        th[first:] = m[first:] = v[first:] = 0.0
        dth, dm, dv = to_dev(th, so), to_dev(m, so), to_dev(v, so)
        pb = torch.zeros(P + po + 8, dtype=torch.bfloat16, device="cuda")[po: po + P]
        go = empty_f32(P, so)
        zr.zr_reduce_scatter_adam(plan, 0, -1, k, dreps, dth, dm, dv, pb, go, step=3, **HP)
        out = empty_f32(P, so)
        zr.zr_reduce_scatter_local(plan, 0, -1, k, dreps, [out])
        assert_bits_equal(host_f32(go), want_g[k], f"fused grad, rank {k}")
        assert_bits_equal(host_f32(out), want_g[k], f"reduced grad, rank {k}")
        w_th, w_m, w_v = adam_oracle(want_g[k], th, m, v, step=3, **HP)
        got_th = host_f32(dth)
        assert_within(got_th, w_th, what=f"master, rank {k}")
        assert_within(host_f32(dm), w_m, what=f"m, rank {k}")
        assert_within(host_f32(dv), w_v, atol=0.0, what=f"v, rank {k}")
        assert np.array_equal(host_u16(pb), bf16_rne_oracle(got_th)), f"bf16 param, rank {k}"


@pytest.mark.parametrize("is_bf16", [True, False])
def test_ipg_random_and_integer(is_bf16):
    numels = [4096 * 2 + 3, 5, 11111, 1, 777]
    plan = zr.zr_plan_buckets(numels, [0] * 5, [(2, 1)], 1 << 20)
    ref = plan_oracle(numels, [0] * 5, [(2, 1)], 1 << 20)
    offsets = ref.param_offset
    rng = np.random.default_rng(5)
    for base, length in [(0, ref.groups[0].padded), (3, 9000), (8196, 11111 + 5)]:
        mg = np.zeros(length, np.float32)
        dmg = to_dev(mg)
        for mb in range(4):
            if mb % 2:
                ints = rng.integers(-256, 257, size=sum(numels)).astype(np.float32)
                grads = np.split(ints, np.cumsum(numels)[:-1])
                if is_bf16:
                    grads = [(x.view(np.uint32) >> 16).astype(np.uint16) for x in grads]
            else:
                grads = [_draw(rng, n, is_bf16) for n in numels]
            ipg_accumulate_oracle(mg, base, offsets, list(range(5)), grads, is_bf16)
            zr.zr_ipg_accumulate(plan, list(range(5)), [to_dev(x, mb % 3) for x in grads],
                                 dmg, window_base=base)
        assert_bits_equal(host_f32(dmg), mg, f"window {base}+{length}")


@pytest.mark.parametrize("is_bf16", [True, False])
def test_ipg_many_params_several_launches(is_bf16):
    """130 params in one call: more segments than one launch carries (48), so
    the call spans three launches and each workgroup's segment search runs
    at full depth; params listed in shuffled order, windows clipping params
    at both ends, gradient pointers misaligned by 0-3 elements."""
    rng = np.random.default_rng(11 + int(is_bf16))
    numels = [int(x) for x in rng.integers(1, 6000, size=130)]
    numels[7] = 40000                                   # several tiles in one segment
    n = len(numels)
    plan = zr.zr_plan_buckets(numels, [0] * n, [(4, 1)], 1 << 30)
    ref = plan_oracle(numels, [0] * n, [(4, 1)], 1 << 30)
    ids = [int(i) for i in rng.permutation(n)]
    total = ref.groups[0].padded
    for base, length in [(0, total), (12345, total // 2), (total - 70001, 70001)]:
        mg = np.zeros(length, np.float32)
        dmg = to_dev(mg)
        for mb in range(3):
            grads = [_draw(rng, numels[p], is_bf16) for p in ids]
            ipg_accumulate_oracle(mg, base, ref.param_offset, ids, grads, is_bf16)
            zr.zr_ipg_accumulate(plan, ids, [to_dev(x, (i + mb) % 4) for i, x in enumerate(grads)],
                                 dmg, window_base=base)
        assert_bits_equal(host_f32(dmg), mg, f"window {base}+{length}")


@pytest.mark.parametrize("sp", [1, 2])
def test_two_replica_reduce_on_every_bf16_pair(sp):
    """Two bf16 replicas holding every pair (a, b) of bf16 bit patterns (2^32
    elements, drawn on the device in chunks), reduced with divisor 2 (sp 1) or
    1 (sp 2): both partitions equal the oracle's rank-order pre-divided sum
    bit for bit, subnormals, infinities and NaNs included."""
    import os
    from concurrent.futures import ThreadPoolExecutor
    from oracle.ipg import widen_bf16
    from oracle.reduce import rank_order_mean
    chunk = 1 << 28
    plan = zr.zr_plan_buckets([chunk], [0], [(2, sp)], 1 << 30)
    P = zr.zr_plan_group_info(plan, 0)[2]
    D = 2 // sp
    outs = [torch.empty(P, device="cuda") for _ in range(2)]
    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    piece = chunk // threads

    def as_bf16(v):
        return torch.where(v >= (1 << 15), v - (1 << 16), v).to(torch.int16).view(torch.bfloat16)

    for c in range((1 << 32) // chunk):
        idx = torch.arange(c * chunk, (c + 1) * chunk, dtype=torch.int64, device="cuda")
        reps = [as_bf16(idx >> 16), as_bf16(idx & 0xFFFF)]
        del idx
        zr.zr_reduce_scatter_local(plan, 0, -1, -1, reps, outs)
        got = np.concatenate([host_f32(o) for o in outs])
        idx_h = np.arange(c * chunk, (c + 1) * chunk, dtype=np.uint64)

        def check(i):
            a, b = i * piece, (i + 1) * piece
            hi = (idx_h[a:b] >> np.uint64(16)).astype(np.uint16)
            lo = (idx_h[a:b] & np.uint64(0xFFFF)).astype(np.uint16)
            with np.errstate(all="ignore"):     # inf - inf and NaN inputs are part of the sweep
                want = rank_order_mean([widen_bf16(hi), widen_bf16(lo)], D)
            assert_bits_equal(got[a:b], want, f"pairs chunk {c} piece {i}")

        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(check, range(threads)))
        del reps


def test_ipg_on_every_bf16_pair():
    """IPG with main_grad holding every bf16 value widened to fp32 against a
    gradient holding every bf16 value (2^32 pairs, on the device in chunks):
    main_grad + widen(grad) equals the oracle's IPG bit for bit."""
    import os
    from concurrent.futures import ThreadPoolExecutor
    from oracle.ipg import widen_bf16
    chunk = 1 << 28
    plan = zr.zr_plan_buckets([chunk], [0], [(2, 1)], 1 << 30)
    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    piece = chunk // threads

    def as_bf16(v):
        return torch.where(v >= (1 << 15), v - (1 << 16), v).to(torch.int16).view(torch.bfloat16)

    for c in range((1 << 32) // chunk):
        idx = torch.arange(c * chunk, (c + 1) * chunk, dtype=torch.int64, device="cuda")
        mg = as_bf16(idx >> 16).float()
        g = as_bf16(idx & 0xFFFF)
        del idx
        zr.zr_ipg_accumulate(plan, [0], [g], mg)
        got = host_f32(mg)
        idx_h = np.arange(c * chunk, (c + 1) * chunk, dtype=np.uint64)

        def check(i):
            a, b = i * piece, (i + 1) * piece
            want = widen_bf16((idx_h[a:b] >> np.uint64(16)).astype(np.uint16)).copy()
            lo = (idx_h[a:b] & np.uint64(0xFFFF)).astype(np.uint16)
            with np.errstate(all="ignore"):
                ipg_accumulate_oracle(want, 0, [0], [0], [lo], True)
            assert_bits_equal(got[a:b], want, f"ipg pairs chunk {c} piece {i}")

        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(check, range(threads)))
        del mg, g


@pytest.mark.parametrize("n,chunk", [(8, 4096 * 3 + 5), (3, 1000), (2, 1)])
def test_ring_steps(n, chunk):
    rng = np.random.default_rng(n)
    bufs = [rng.standard_normal(n * chunk).astype(np.float32) for _ in range(n)]
    dev = [to_dev(b) for b in bufs]
    for s in range(n - 1):
        zr.zr_ring_rs_step(dev, chunk, s)
    want, _ = ring_reduce_scatter_oracle(bufs)
    for k in range(n):
        got = host_f32(dev[k])
        assert_bits_equal(got, want[k], f"rank {k}")
        assert_bits_equal(got[k * chunk:(k + 1) * chunk], ring_order_sum(bufs, k))


def test_ring_integer_equals_direct_sum():
    n, chunk = 8, 5000
    rng = np.random.default_rng(0)
    bufs = [rng.integers(-1000, 1000, size=n * chunk).astype(np.float32) for _ in range(n)]
    dev = [to_dev(b) for b in bufs]
    for s in range(n - 1):
        zr.zr_ring_rs_step(dev, chunk, s)
    total = sum(b.astype(np.int64) for b in bufs).astype(np.float32)
    for k in range(n):
        assert np.array_equal(host_f32(dev[k])[k * chunk:(k + 1) * chunk],
                              total[k * chunk:(k + 1) * chunk])


def test_copy_grads_in_partition():
    """Standalone copy into the partition against the copy oracle, on a
    shrunken MoE-like list (interleaved groups, many small buckets): the
    bucket-layout source is the oracle's reduced bucket, so the copied
    partition also equals the oracle's reduce-scatter of that bucket."""
    w = workloads.get("moe-16l")
    numels = [n // 4096 + 1 for n in w.numels[:34]]
    pg = w.param_groups[:34]
    ref = plan_oracle(numels, pg, w.groups, 3000)
    plan = zr.zr_plan_buckets(numels, pg, w.groups, 3000)
    rng = np.random.default_rng(1)
    reps = [[rng.standard_normal(g.total).astype(np.float32) for _ in range(g.world)]
            for g in ref.groups]
    for b in range(ref.num_buckets):
        src = np.zeros(3000, np.float32)
        lay = bucket_layout_mean(ref, b, reps, False)
        src[:lay.size] = lay
        dsrc = to_dev(src, b % 2)
        for g, info in enumerate(ref.groups):
            for k in range(info.world):
                out = empty_f32(info.part_numel)
                zr.zr_copy_grads_in_partition(plan, g, b, k, dsrc, out)
                want = copy_grads_in_partition_oracle(ref, g, b, k, src)
                assert_bits_equal(host_f32(out), want, f"bucket {b} group {g} dst {k}")
                rs = reduce_scatter_oracle(ref, g, reps[g], False, bucket=b, dst=k)[k]
                sel = ~np.isnan(want)
                assert_bits_equal(host_f32(out)[sel], rs[sel], f"bucket {b} group {g} dst {k} vs RS")


def test_invalid_call_leaves_outputs_untouched():
    plan = zr.zr_plan_buckets([100], [0], [(2, 1)], 64)
    reps = [to_dev(np.ones(100, np.float32)) for _ in range(2)]
    out = empty_f32(50, fill=7.0)
    short = [(to_dev(np.ones(10, np.float32)), 0)] * 2
    with pytest.raises(zr.ZrError):
        zr.zr_reduce_scatter_local(plan, 0, -1, 0, short, [out])
    assert (host_f32(out) == 7.0).all()
    zr.zr_reduce_scatter_local(plan, 0, -1, 0, reps, [out])
    assert (host_f32(out) == 1.0).all()


@pytest.mark.parametrize("R,sp,is_bf16", [(64, 1, False), (64, 4, True), (17, 1, True), (7, 7, False)])
def test_large_and_odd_replica_counts(R, sp, is_bf16):
    # R = 64 is the largest world a plan accepts; 17 and 7 take the run-time
    # replica loop; D = 64, 16, 17 and 1.
    numels = [4096 * 3 + 11, 5, 3000]
    ref = plan_oracle(numels, [0] * 3, [(R, sp)], 7000)
    plan = zr.zr_plan_buckets(numels, [0] * 3, [(R, sp)], 7000)
    info = ref.groups[0]
    rng = np.random.default_rng(R)
    reps = [_draw(rng, info.total, is_bf16, sigma=0.1) for _ in range(R)]
    want = reduce_scatter_oracle(ref, 0, reps, is_bf16)
    outs = [empty_f32(info.part_numel) for _ in range(R)]
    zr.zr_reduce_scatter_local(plan, 0, -1, -1, [to_dev(x) for x in reps], outs)
    for k in range(R):
        assert_bits_equal(host_f32(outs[k]), want[k], f"R={R} dst {k}")
    # fused on the last partition (it holds the padding)
    k = R - 1
    P = info.part_numel
    th = (rng.standard_normal(P) * 0.02).astype(np.float32)
    th[max(0, info.total - k * P):] = 0.0
    z = np.zeros(P, np.float32)
    dth, dm, dv = to_dev(th), to_dev(z), to_dev(z)
    g = empty_f32(P)
    zr.zr_reduce_scatter_adam(plan, 0, -1, k, [to_dev(x) for x in reps], dth, dm, dv, None, g, **HP)
    assert_bits_equal(host_f32(g), want[k], "fused grad")
    w_th, w_m, w_v = adam_oracle(want[k], th, z, z, step=1, **HP)
    assert_within(host_f32(dth), w_th, what="master")


# Partition size 2 (mod 4) with align 1 puts odd ranks' bf16 replica windows
# 4 bytes off the state buffers' 16-byte grid, and state offsets of 1-3
# elements leave the fp32 streams dword- but not 16-byte-aligned: no phase is
# slot-aligned for every stream, so the host launches the kernel variant that
# also accepts dword-aligned phases, and reads bf16 replicas an odd number of
# elements off with shifted loads.  Every rank, several tiles, against the
# oracle.
@pytest.mark.parametrize("is_bf16", [True, False])
@pytest.mark.parametrize("state_off,pb_off", [(0, 0), (1, 2), (2, 1), (3, 3)])
@pytest.mark.parametrize("p_mod", [2, 1, 3])
def test_dword_aligned_phases(is_bf16, state_off, pb_off, p_mod):
    # P = 4096 + p_mod: with P odd, odd ranks' bf16 windows also sit an odd
    # number of elements off, which the variant reads with shifted loads.
    numels = [8 * (4096 + p_mod)]
    ref = plan_oracle(numels, [0], [(8, 1)], 1 << 30)
    plan = zr.zr_plan_buckets(numels, [0], [(8, 1)], 1 << 30)
    info = ref.groups[0]
    P, R, T = info.part_numel, info.world, info.total
    assert P % 4 == p_mod
    rng = np.random.default_rng(100 + state_off)
    reps = [_draw(rng, T, is_bf16, sigma=1e-3) for _ in range(R)]
    dreps = [to_dev(x) for x in reps]
    want = reduce_scatter_oracle(ref, 0, reps, is_bf16)
    for k in range(R):
        th = (rng.standard_normal(P) * 0.02).astype(np.float32)
        m = (rng.standard_normal(P) * 1e-4).astype(np.float32)
        v = np.abs(rng.standard_normal(P) * 1e-8).astype(np.float32)
        first = max(0, min(P, T - k * P))
        th[first:] = m[first:] = v[first:] = 0.0
        dth, dm, dv = to_dev(th, state_off), to_dev(m, state_off), to_dev(v, state_off)
        pb = torch.zeros(P + pb_off + 8, dtype=torch.bfloat16, device="cuda")[pb_off:pb_off + P]
        go = empty_f32(P, state_off)
        zr.zr_reduce_scatter_adam(plan, 0, -1, k, dreps, dth, dm, dv, pb, go, step=2, **HP)
        out = empty_f32(P, state_off)
        zr.zr_reduce_scatter_local(plan, 0, -1, k, dreps, [out])
        assert_bits_equal(host_f32(go), want[k], f"rank {k} fused grad")
        assert_bits_equal(host_f32(out), want[k], f"rank {k} reduced grad")
        w_th, w_m, w_v = adam_oracle(want[k], th, m, v, step=2, **HP)
        got = host_f32(dth)
        assert_within(got, w_th, what=f"rank {k} master")
        assert_within(host_f32(dm), w_m, what=f"rank {k} m")
        assert_within(host_f32(dv), w_v, atol=0.0, what=f"rank {k} v")
        assert np.array_equal(host_u16(pb), bf16_rne_oracle(got)), f"rank {k} bf16"


# Replica counts without a compiled specialization (the rank loop runs at run
# time) with an odd partition size: the bf16 replicas of odd ranks sit an odd
# number of elements off and are read with shifted loads inside that loop.
@pytest.mark.parametrize("R", [5, 12])
def test_dword_phases_runtime_replica_count(R):
    P = 2 * 4096 + 1
    numels = [R * P - 3]
    ref = plan_oracle(numels, [0], [(R, 1)], 1 << 30)
    plan = zr.zr_plan_buckets(numels, [0], [(R, 1)], 1 << 30)
    info = ref.groups[0]
    assert info.part_numel == P and P % 2 == 1
    T = info.total
    rng = np.random.default_rng(R)
    reps = [_draw(rng, T, True, sigma=1e-3) for _ in range(R)]
    dreps = [to_dev(x) for x in reps]
    want = reduce_scatter_oracle(ref, 0, reps, True)
    for k in range(R):
        th = (rng.standard_normal(P) * 0.02).astype(np.float32)
        first = max(0, min(P, T - k * P))
        th[first:] = 0.0
        z = np.zeros(P, np.float32)
        dth, dm, dv = to_dev(th), to_dev(z), to_dev(z)
        pb = torch.zeros(P, dtype=torch.bfloat16, device="cuda")
        go = empty_f32(P)
        zr.zr_reduce_scatter_adam(plan, 0, -1, k, dreps, dth, dm, dv, pb, go, **HP)
        assert_bits_equal(host_f32(go), want[k], f"rank {k} fused grad")
        w_th, w_m, w_v = adam_oracle(want[k], th, z, z, step=1, **HP)
        got = host_f32(dth)
        assert_within(got, w_th, what=f"rank {k} master")
        assert_within(host_f32(dm), w_m, what=f"rank {k} m")
        assert_within(host_f32(dv), w_v, atol=0.0, what=f"rank {k} v")
        assert np.array_equal(host_u16(pb), bf16_rne_oracle(got)), f"rank {k} bf16"


@pytest.mark.parametrize("is_bf16", [True, False])
def test_ipg_first_micro_batch_equals_add_into_zeros(is_bf16):
    """zr_ipg_accumulate_first (the step's first micro-batch, main_grad not
    read) against zr_ipg_accumulate into a zeroed window and the oracle's IPG
    from zeros, bit for bit: -0 and special values among the gradients,
    windows clipping params at both ends, gradient and main_grad pointers off
    by 0-3 elements (the dword-aligned variant included); elements no listed
    param covers keep what the window held; later micro-batches accumulate
    onto the first one's result."""
    rng = np.random.default_rng(21 + int(is_bf16))
    numels = [4096 * 3 + 5, 1, 700, 33, 20000, 6]
    n = len(numels)
    plan = zr.zr_plan_buckets(numels, [0] * n, [(2, 1)], 1 << 30)
    ref = plan_oracle(numels, [0] * n, [(2, 1)], 1 << 30)
    total = ref.groups[0].padded
    listed = [0, 2, 3, 4]                       # params 1 and 5 are not listed
    specials = np.array([-0.0, 0.0, np.inf, -np.inf, np.nan, 1e-40, -1e-40, 3e38],
                        np.float32)
    for base, length, off_g, off_mg in [(0, total, 0, 0), (7, 15000, 1, 3),
                                        (12290, total - 12290 - 3, 2, 1)]:
        grads = []
        for p in listed:
            x = (rng.standard_normal(numels[p]) * 1e-3).astype(np.float32)
            x[: min(len(specials), numels[p])] = specials[: min(len(specials), numels[p])]
            if is_bf16:
                x = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
            grads.append(x)
        fill = rng.standard_normal(length).astype(np.float32)
        got = to_dev(fill, off_mg)
        zr.zr_ipg_accumulate_first(plan, listed, [to_dev(x, off_g) for x in grads], got,
                                   window_base=base)
        zeros = to_dev(np.zeros(length, np.float32), off_mg)
        zr.zr_ipg_accumulate(plan, listed, [to_dev(x, off_g) for x in grads], zeros,
                             window_base=base)
        want = np.zeros(length, np.float32)
        ipg_accumulate_oracle(want, base, ref.param_offset, listed, grads, is_bf16)
        covered = np.zeros(length, bool)
        for p in listed:
            lo = max(ref.param_offset[p], base) - base
            hi = min(ref.param_offset[p] + numels[p], base + length) - base
            if hi > lo:
                covered[lo:hi] = True
        g = host_f32(got)
        assert_bits_equal(g[covered], want[covered], "first micro-batch vs oracle")
        assert_bits_equal(g[covered], host_f32(zeros)[covered], "first vs add into zeros")
        assert_bits_equal(g[~covered], fill[~covered], "elements no listed param covers")
        # a second micro-batch accumulates onto the first one's result
        grads2 = [_draw(rng, numels[p], is_bf16) for p in listed]
        zr.zr_ipg_accumulate(plan, listed, [to_dev(x, off_g) for x in grads2], got,
                             window_base=base)
        ipg_accumulate_oracle(want, base, ref.param_offset, listed, grads2, is_bf16)
        assert_bits_equal(host_f32(got)[covered], want[covered], "second micro-batch")
