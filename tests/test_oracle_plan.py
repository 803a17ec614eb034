"""Pins for oracle O1 (the plan): a hand-derived worked example, the
brute-force element map, tiling invariants and closed-form sizes."""

import os
import random

import pytest

from oracle.plan import plan_oracle, plan_bruteforce, slices_for
from zero_partition_aware_amd import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tiny_plan.txt")


def _read_golden():
    totals, params, slices = None, [], []
    with open(GOLDEN) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            tag, *rest = line.split()
            if tag == "totals":
                totals = tuple(int(x) for x in rest)
            elif tag == "param":
                pid, off, ids, gso = rest
                params.append((int(pid), int(off),
                               [int(x) for x in ids.split(";")],
                               [int(x) for x in gso.split(";")]))
            elif tag == "slice":
                slices.append(tuple(int(x) for x in rest))
    return totals, params, slices


def test_tiny_plan_matches_hand_derivation():
    w = workloads.get("tiny")
    for build in (plan_oracle, plan_bruteforce):
        plan = build(w.numels, w.param_groups, w.groups, w.reduce_bucket_size)
        totals, params, slices = _read_golden()
        gi = plan.groups[0]
        assert (gi.total, gi.padded, gi.part_numel, plan.num_buckets) == totals
        for pid, off, ids, gso in params:
            assert plan.param_offset[pid] == off
            assert plan.param_to_partition_ids[pid] == ids
            assert [plan.grad_start_offset[pid][k] for k in ids] == gso
        got = [(s.bucket, s.dst, s.bucket_offset, s.flat_offset,
                s.part_offset, s.numel) for s in plan.slices]
        assert got == slices


def _random_case(rng):
    n_groups = rng.choice([1, 1, 2, 3])
    groups = []
    for _ in range(n_groups):
        sp = rng.choice([1, 1, 2, 3])
        groups.append((sp * rng.randint(1, 5), sp))
    n_params = rng.randint(1, 12)
    numels = [rng.choice([1, 2, 3, rng.randint(1, 90)]) for _ in range(n_params)]
    pg = [rng.randrange(n_groups) for _ in range(n_params)]
    B = rng.choice([1, 2, 5, 7, 31, 100, 10_000])
    align = rng.choice([1, 1, 2, 4, 8])
    return numels, pg, groups, B, align


def test_interval_plan_equals_bruteforce_random():
    rng = random.Random(1234)
    for _ in range(400):
        numels, pg, groups, B, align = _random_case(rng)
        a = plan_oracle(numels, pg, groups, B, align)
        b = plan_bruteforce(numels, pg, groups, B, align)
        assert a.slices == b.slices
        assert a.param_offset == b.param_offset
        assert a.param_to_partition_ids == b.param_to_partition_ids
        assert a.grad_start_offset == b.grad_start_offset
        assert a.num_buckets == b.num_buckets
        for ga, gb in zip(a.groups, b.groups):
            assert ga == gb


def _check_invariants(plan):
    B = plan.reduce_bucket_size
    # Slices tile the buckets in order, each non-last bucket holding exactly B.
    per_bucket = {}
    for s in plan.slices:
        per_bucket.setdefault(s.bucket, []).append(s)
    total = sum(g.total for g in plan.groups)
    assert sorted(per_bucket) == list(range(plan.num_buckets))
    for b, ss in per_bucket.items():
        pos = 0
        for s in ss:
            assert s.bucket_offset == pos
            pos += s.numel
        if b < plan.num_buckets - 1:
            assert pos == B
        else:
            assert pos == total - B * (plan.num_buckets - 1)
    # Every flat element of every group lies in exactly one slice, and each
    # destination receives P elements minus padding.
    for g, info in enumerate(plan.groups):
        covered = [0] * info.total
        per_dst = [0] * info.world
        for s in slices_for(plan, g):
            assert s.flat_offset == s.dst * info.part_numel + s.part_offset
            assert 0 <= s.part_offset and s.part_offset + s.numel <= info.part_numel
            for f in range(s.flat_offset, s.flat_offset + s.numel):
                covered[f] += 1
            per_dst[s.dst] += s.numel
        assert all(c == 1 for c in covered)
        P = info.part_numel
        assert per_dst == [min(P, max(0, info.total - k * P))
                           for k in range(info.world)]
        assert info.padded % info.world == 0
        assert info.divisor * info.sp == info.world
    # Adjacent slices never share (bucket, group, dst): they are maximal.
    for s, t in zip(plan.slices, plan.slices[1:]):
        assert (s.bucket, s.group, s.dst) != (t.bucket, t.group, t.dst)


def test_plan_invariants_random():
    rng = random.Random(99)
    for _ in range(300):
        numels, pg, groups, B, align = _random_case(rng)
        _check_invariants(plan_oracle(numels, pg, groups, B, align))


def test_align_pads_partition_to_multiple():
    plan = plan_oracle([10, 3], [0, 0], [(4, 1)], 5, align=8)
    g = plan.groups[0]
    assert (g.total, g.padded, g.part_numel) == (13, 32, 8)


@pytest.mark.parametrize("name,T,P,nb,nslices", [
    ("gpt2-small", 124_439_808, 15_554_976, 1, 8),
])
def test_workload_closed_forms_single_group(name, T, P, nb, nslices):
    w = workloads.get(name)
    plan = plan_oracle(w.numels, w.param_groups, w.groups, w.reduce_bucket_size)
    assert len(w.numels) == 148
    assert plan.groups[0].total == T
    assert plan.groups[0].part_numel == P
    assert plan.num_buckets == nb
    assert len(plan.slices) == nslices


def test_llama_closed_forms():
    w = workloads.get("llama3-8b")
    assert len(w.numels) == 291
    plan = plan_oracle(w.numels, w.param_groups, w.groups, w.reduce_bucket_size)
    g = plan.groups[0]
    assert g.total == 8_030_261_248
    assert g.padded == g.total          # already a multiple of 8
    assert g.part_numel == 1_003_782_656
    assert plan.num_buckets == 17
    last = sum(s.numel for s in plan.slices if s.bucket == 16)
    assert last == 8_030_261_248 - 16 * 500_000_000 == 30_261_248
    for k in range(8):
        assert sum(s.numel for s in slices_for(plan, 0, dst=k)) == g.part_numel


def test_moe_closed_forms():
    w = workloads.get("moe-16l")
    assert len(w.numels) == 272
    plan = plan_oracle(w.numels, w.param_groups, w.groups, w.reduce_bucket_size)
    dense, expert = plan.groups
    assert (dense.total, dense.part_numel, dense.divisor) == \
        (268_959_744, 33_619_968, 4)
    assert (expert.total, expert.part_numel, expert.divisor) == \
        (1_074_069_504, 537_034_752, 1)
    assert plan.num_buckets == 269
    # A bucket carries both groups exactly when a dense<->expert transition of
    # the list falls strictly inside it: 16 + 15 transitions along the list.
    pos, transitions = 0, []
    for i, n in enumerate(w.numels):
        if i and w.param_groups[i] != w.param_groups[i - 1]:
            transitions.append(pos)
        pos += n
    assert len(transitions) == 31
    inside = {t // w.reduce_bucket_size for t in transitions
              if t % w.reduce_bucket_size}
    both = {b for b in range(plan.num_buckets)
            if {s.group for s in plan.slices if s.bucket == b} == {0, 1}}
    assert both == inside and len(both) == 31


@pytest.mark.parametrize("args", [
    dict(numels=[0], pg=[0], groups=[(2, 1)], B=4),
    dict(numels=[3], pg=[1], groups=[(2, 1)], B=4),
    dict(numels=[3], pg=[0], groups=[(3, 2)], B=4),
    dict(numels=[3], pg=[0], groups=[(0, 1)], B=4),
    dict(numels=[3], pg=[0], groups=[(2, 1)], B=0),
])
def test_plan_rejects_invalid(args):
    with pytest.raises(ValueError):
        plan_oracle(args["numels"], args["pg"], args["groups"], args["B"])
