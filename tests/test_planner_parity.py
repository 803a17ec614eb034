"""The C++ planner (libzr, zr_plan_buckets and its queries) against the
oracle's plan: identical slices, offsets, partition ids, grad start offsets
and group sizes on random lists and on the full workload lists."""

import random

import pytest

from oracle.plan import plan_oracle
from tests._lib import load
from zero_partition_aware_amd import workloads

zr = load()


def _compare(numels, pg, groups, B, align):
    ref = plan_oracle(numels, pg, groups, B, align)
    plan = zr.zr_plan_buckets(numels, pg, groups, B, 0, align)
    assert zr.zr_plan_num_buckets(plan) == ref.num_buckets
    assert zr.zr_plan_num_params(plan) == len(numels)
    for g, info in enumerate(ref.groups):
        t, L, P, d = zr.zr_plan_group_info(plan, g)
        assert (t, L, P, d) == (info.total, info.padded, info.part_numel,
                                float(info.divisor))
    want = [(s.bucket, s.group, s.dst, s.bucket_offset, s.flat_offset,
             s.part_offset, s.numel) for s in ref.slices]
    assert zr.zr_plan_slices(plan, -1) == want
    by_bucket = {}
    for w in want:
        by_bucket.setdefault(w[0], []).append(w)
    nb = ref.num_buckets
    sample = range(nb) if nb <= 64 else sorted({0, nb - 1, *random.Random(nb).sample(range(nb), 62)})
    for b in sample:
        assert zr.zr_plan_slices(plan, b) == by_bucket[b]
    for p in range(len(numels)):
        assert zr.zr_plan_param_offset(plan, p) == ref.param_offset[p]
        ids = zr.zr_plan_param_partitions(plan, p)
        assert ids == ref.param_to_partition_ids[p]
        for k in ids:
            assert zr.zr_plan_grad_start_offset(plan, p, k) == ref.grad_start_offset[p][k]
    return plan


def test_random_lists_match_oracle():
    rng = random.Random(2024)
    for _ in range(500):
        ng = rng.choice([1, 1, 2, 3])
        groups = []
        for _ in range(ng):
            sp = rng.choice([1, 2, 4])
            groups.append((sp * rng.randint(1, 8), sp))
        n = rng.randint(1, 40)
        numels = [rng.choice([1, 2, 7, rng.randint(1, 5000)]) for _ in range(n)]
        pg = [rng.randrange(ng) for _ in range(n)]
        B = rng.choice([1, 3, 64, 1000, 4096, 1 << 20])
        align = rng.choice([1, 1, 4, 8, 16])
        _compare(numels, pg, groups, B, align)


@pytest.mark.parametrize("name", ["tiny", "gpt2-small", "llama3-8b", "moe-16l"])
def test_workload_plans_match_oracle(name):
    w = workloads.get(name)
    _compare(w.numels, w.param_groups, w.groups, w.reduce_bucket_size, 1)


def test_huge_bucket_size_and_stage_flag():
    plan = zr.zr_plan_buckets([5, 6], [0, 0], [(2, 1)], (1 << 62), 1, 1)
    assert zr.zr_plan_num_buckets(plan) == 1
    assert zr.zr_plan_partition_gradients(plan) == 1


@pytest.mark.parametrize("numels,pg,groups,B,align,msg", [
    ([0], [0], [(2, 1)], 4, 1, "numel"),
    ([3], [1], [(2, 1)], 4, 1, "group index"),
    ([3], [0], [(3, 2)], 4, 1, "divide"),
    ([3], [0], [(0, 1)], 4, 1, "positive"),
    ([3], [0], [(65, 1)], 4, 1, "ZR_MAX_WORLD"),
    ([3], [0], [(2, 1)], 0, 1, "reduce_bucket_size"),
    ([3], [0], [(2, 1)], 4, 0, "align"),
    ([(1 << 62), (1 << 62)], [0, 0], [(2, 1)], 4, 1, "overflow"),
    ([(1 << 62) + 1], [0], [(2, 1)], 4, 1 << 62, "overflow"),
])
def test_invalid_plans_are_rejected(numels, pg, groups, B, align, msg):
    with pytest.raises(zr.ZrError) as ei:
        zr.zr_plan_buckets(numels, pg, groups, B, 0, align)
    assert ei.value.status == zr.ZR_ERR_INVALID
    assert msg in str(ei.value)


def test_query_errors():
    plan = zr.zr_plan_buckets([37, 2112, 129], [0, 0, 0], [(4, 1)], 1000)
    with pytest.raises(zr.ZrError):
        zr.zr_plan_grad_start_offset(plan, 0, 1)     # p0 lies in partition 0 only
    with pytest.raises(zr.ZrError):
        zr.zr_plan_param_offset(plan, 3)
    with pytest.raises(zr.ZrError):
        zr.zr_plan_slices(plan, 3)
    with pytest.raises(zr.ZrError):
        zr.zr_plan_group_info(plan, 1)


def test_param_buckets_match_list_positions():
    rng = random.Random(7)
    for _ in range(100):
        n = rng.randint(1, 30)
        numels = [rng.randint(1, 3000) for _ in range(n)]
        pg = [rng.randrange(2) for _ in range(n)]
        B = rng.choice([1, 100, 2999, 10 ** 6])
        ref = plan_oracle(numels, pg, [(2, 1), (4, 2)], B)
        plan = zr.zr_plan_buckets(numels, pg, [(2, 1), (4, 2)], B)
        pos = 0
        for p, ne in enumerate(numels):
            first, last = zr.zr_plan_param_buckets(plan, p)
            assert (first, last) == (pos // B, (pos + ne - 1) // B)
            # every bucket in that range holds a slice of this param
            mine = {s.bucket for s in ref.slices if s.group == pg[p] and
                    s.flat_offset < ref.param_offset[p] + ne and
                    s.flat_offset + s.numel > ref.param_offset[p]}
            assert mine == set(range(first, last + 1))
            pos += ne


hypothesis = pytest.importorskip("hypothesis")
st = hypothesis.strategies


@st.composite
def _plans(draw):
    ng = draw(st.integers(1, 3))
    groups = []
    for _ in range(ng):
        sp = draw(st.sampled_from([1, 2, 3, 4]))
        groups.append((sp * draw(st.integers(1, 16 // sp)), sp))
    n = draw(st.integers(1, 60))
    numels = draw(st.lists(st.integers(1, 100000), min_size=n, max_size=n))
    pg = draw(st.lists(st.integers(0, ng - 1), min_size=n, max_size=n))
    total = sum(numels)
    lo = max(1, total // 20000)                 # at most ~20,000 buckets
    B = draw(st.one_of(st.integers(lo, lo + 63), st.integers(lo, 2 * total)))
    align = draw(st.sampled_from([1, 2, 4, 8, 16, 64]))
    return numels, pg, groups, B, align


@hypothesis.settings(max_examples=200, deadline=None, derandomize=True,
                     suppress_health_check=list(hypothesis.HealthCheck))
@hypothesis.given(_plans())
def test_planner_matches_oracle_on_generated_plans(case):
    """Property form of the comparison above (the planner equals the oracle on
    every drawn list); a counterexample is shrunk to a minimal plan."""
    _compare(*case)
