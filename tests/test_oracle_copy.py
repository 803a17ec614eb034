"""Pins for the copy_grads_in_partition oracle: the hand-derived tiny plan fixes
where every element of a bucket lands, and a bucket-layout reduction followed
by the copy must equal the direct partition reduce-scatter, for every bucket,
group and destination of random plans (two independent routes to the same
partition).  Planted mistakes in the copy are caught."""

import random

import numpy as np
import pytest

from oracle import copy as copy_mod
from oracle.copy import bucket_layout_mean, copy_grads_in_partition_oracle
from oracle.plan import plan_oracle
from oracle.reduce import reduce_scatter_oracle
from tests.test_oracle_plan import _read_golden
from zero_partition_aware_amd import workloads


def _golden_pin(copy_fn):
    """Tiny workload: a bucket-layout source holding its own bucket offsets
    (0, 1, 2, ...) must land exactly where the hand-derived slices say."""
    w = workloads.get("tiny")
    plan = plan_oracle(w.numels, w.param_groups, w.groups, w.reduce_bucket_size)
    (T, L, P, nb), _, slices = _read_golden()
    for b in range(nb):
        src = np.arange(w.reduce_bucket_size, dtype=np.float32)
        for k in range(4):
            got = copy_fn(plan, 0, b, k, src)
            want = np.full(P, np.nan, np.float32)
            for (sb, sd, boff, _flat, poff, n) in slices:
                if sb == b and sd == k:
                    want[poff:poff + n] = np.arange(boff, boff + n, dtype=np.float32)
            assert np.array_equal(np.isnan(got), np.isnan(want)), (b, k)
            assert np.array_equal(got[~np.isnan(got)], want[~np.isnan(want)]), (b, k)


def _composition_pin(copy_fn, seeds=range(40)):
    """bucket-layout mean, then copy == the partition reduce-scatter of that
    bucket (bitwise on every element the copy writes), and the copies of all
    buckets together write every real element of every partition once."""
    for seed in seeds:
        rng = random.Random(seed)
        groups = [(rng.choice([1, 2, 3, 4, 8]), 1) for _ in range(rng.choice([1, 2]))]
        n = rng.randint(1, 8)
        numels = [rng.randint(1, 3000) for _ in range(n)]
        pg = [rng.randrange(len(groups)) for _ in range(n)]
        B = rng.choice([7, 100, 999, 5000])
        plan = plan_oracle(numels, pg, groups, B)
        nprng = np.random.default_rng(seed)
        reps = [[nprng.standard_normal(g.total).astype(np.float32) for _ in range(g.world)]
                for g in plan.groups]
        written = [np.zeros(g.padded, bool) for g in plan.groups]
        for b in range(plan.num_buckets):
            src = bucket_layout_mean(plan, b, reps, False)
            for g, info in enumerate(plan.groups):
                for k in range(info.world):
                    got = copy_fn(plan, g, b, k, src)
                    want = reduce_scatter_oracle(plan, g, reps[g], False, bucket=b, dst=k)[k]
                    sel = ~np.isnan(got)
                    assert np.array_equal(got[sel].view(np.uint32), want[sel].view(np.uint32)), \
                        (seed, b, g, k)
                    part = written[g][k * info.part_numel:(k + 1) * info.part_numel]
                    assert not (part & sel).any(), "an element written by two buckets"
                    part |= sel
        for g, info in enumerate(plan.groups):
            assert written[g][:info.total].all() and not written[g][info.total:].any()


def test_copy_places_the_hand_derived_slices():
    _golden_pin(copy_grads_in_partition_oracle)


def test_bucket_layout_then_copy_equals_reduce_scatter():
    _composition_pin(copy_grads_in_partition_oracle)


@pytest.mark.parametrize("kind", ["flat_for_bucket_offset", "swap_offsets", "off_by_one",
                                  "all_destinations"])
def test_copy_mutants_are_caught(kind):
    def mutant(plan, group, bucket, dst, src):
        P = plan.groups[group].part_numel
        src = np.asarray(src, np.float32)
        out = np.full(P, np.nan, np.float32)
        for s in plan.slices:
            if s.group != group or s.bucket != bucket:
                continue
            if s.dst != dst and kind != "all_destinations":
                continue
            so = {"flat_for_bucket_offset": s.flat_offset, "swap_offsets": s.part_offset,
                  "off_by_one": s.bucket_offset + 1, "all_destinations": s.bucket_offset}[kind]
            po = s.bucket_offset if kind == "swap_offsets" else s.part_offset
            po = min(po, P - s.numel)
            seg = src[so: so + s.numel]
            out[po: po + seg.size] = seg
        return out
    with pytest.raises(AssertionError):
        _golden_pin(mutant)
        _composition_pin(mutant)


def test_copy_module_names_its_source():
    assert "§三.3" in copy_mod.__doc__
