"""Pins for oracles O3/O4 (pre-divide rank-order reduce-scatter) and the bf16
widening it starts from."""

import random

import numpy as np
import pytest
import torch

from oracle.ipg import widen_bf16
from oracle.plan import plan_oracle
from oracle.reduce import (allreduce_average_oracle, rank_order_mean,
                           reduce_scatter_oracle)
from zero_partition_aware_amd import workloads

F = np.float32


def test_rank_order_is_pinned_by_hand_example():
    # D = 1.  Exact sum is 2; rank order 0..3 gives
    #   fl(2^24 + 1) = 2^24 (tie to even), fl(2^24 + 1) = 2^24, 2^24 - 2^24 = 0;
    # pairwise order would give 1 and reverse order 2.
    vals = [np.array([v], F) for v in (2.0 ** 24, 1.0, 1.0, -(2.0 ** 24))]
    assert rank_order_mean(vals, 1)[0] == 0.0
    assert rank_order_mean(vals[::-1], 1)[0] == 2.0


def test_accumulator_starts_from_rank0_term_keeps_negative_zero():
    vals = [np.array([-0.0], F), np.array([-0.0], F)]
    out = rank_order_mean(vals, 2)
    assert out[0] == 0.0 and np.signbit(out[0])


def test_integer_inputs_exact_against_python_ints():
    rng = np.random.default_rng(5)
    for R, D in [(4, 4), (8, 4), (6, 6), (3, 1), (8, 8)]:
        xs = [rng.integers(-1000, 1000, size=257) * D for _ in range(R)]
        want = [sum(int(x[i]) // D for x in xs) for i in range(257)]
        got = rank_order_mean([x.astype(F) for x in xs], D)
        assert got.tolist() == [float(w) for w in want]


def test_pow2_divisor_mean_equals_sum_over_n_in_normal_range():
    # Averaging gives sum/N: with D a power of two every x/D is exact, so the
    # pre-divided rank-order sum equals the rank-order sum divided once.
    rng = np.random.default_rng(7)
    for D in (1, 2, 4, 8, 16):
        xs = [rng.standard_normal(10_000).astype(F) for _ in range(8)]
        pre = rank_order_mean(xs, D)
        acc = xs[0].copy()
        for x in xs[1:]:
            acc = np.add(acc, x, dtype=F)
        post = np.divide(acc, F(D), dtype=F)
        assert np.array_equal(pre.view(np.uint32), post.view(np.uint32))


def test_single_replica_is_identity():
    x = workloads.host_special_values(3, 500)
    out = rank_order_mean([x], 1)
    same = (out.view(np.uint32) == x.view(np.uint32)) | (np.isnan(out) & np.isnan(x))
    assert same.all()


def test_predivide_avoids_overflow_of_sum_first():
    xs = [np.array([3e38], F)] * 4
    pre = rank_order_mean(xs, 4)
    assert np.isfinite(pre[0]) and pre[0] == F(3e38)
    with np.errstate(over="ignore"):
        s = xs[0] + xs[1] + xs[2] + xs[3]
    assert np.isinf(s[0])


def test_subnormals_are_kept():
    # 2^-140 / 4 = 2^-142, a subnormal; flushing would give 0.
    x = np.array([2.0 ** -140], F)
    out = rank_order_mean([x, x, x, x], 4)
    assert out[0] == F(2.0 ** -140)


def test_widen_bf16_matches_torch():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    mine = widen_bf16(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    same = (mine.view(np.uint32) == ref.view(np.uint32)) | (np.isnan(mine) & np.isnan(ref))
    assert same.all()


def _random_plan(rng):
    R = rng.choice([1, 2, 3, 4, 8])
    sp = rng.choice([d for d in (1, 2, 4) if R % d == 0])
    numels = [rng.randint(1, 60) for _ in range(rng.randint(1, 8))]
    return numels, [0] * len(numels), [(R, sp)]


@pytest.mark.parametrize("is_bf16", [False, True])
def test_concatenated_shards_equal_allreduce(is_bf16):
    rng = random.Random(11)
    nrng = np.random.default_rng(11)
    for _ in range(60):
        numels, pg, groups = _random_plan(rng)
        B = rng.choice([1, 3, 7, 50, 1000])
        plan = plan_oracle(numels, pg, groups, B)
        info = plan.groups[0]
        T = info.total
        if is_bf16:
            reps = [nrng.integers(0, 1 << 16, size=T).astype(np.uint16) for _ in range(info.world)]
            reps = [np.where(np.isnan(widen_bf16(r)), 0, r).astype(np.uint16) for r in reps]
        else:
            reps = [nrng.standard_normal(T).astype(F) for _ in range(info.world)]
        shards = reduce_scatter_oracle(plan, 0, reps, is_bf16)
        full = np.concatenate([shards[k] for k in range(info.world)])
        ar = allreduce_average_oracle(reps, info.divisor, is_bf16)
        with np.errstate(all="ignore"):
            assert np.array_equal(full[:T].view(np.uint32), ar.view(np.uint32))
        assert (full[T:] == 0).all()


def test_bucket_size_does_not_change_shards():
    rng = np.random.default_rng(2)
    w = workloads.get("tiny")
    reps = [rng.standard_normal(2278).astype(F) for _ in range(4)]
    ref = None
    for B in (1, 7, 1000, 1 << 40):
        plan = plan_oracle(w.numels, w.param_groups, w.groups, B)
        shards = reduce_scatter_oracle(plan, 0, reps, False)
        got = np.concatenate([shards[k] for k in range(4)]).view(np.uint32)
        if ref is None:
            ref = got
        assert np.array_equal(got, ref)


def test_per_bucket_calls_compose_to_whole():
    rng = np.random.default_rng(4)
    w = workloads.get("tiny")
    plan = plan_oracle(w.numels, w.param_groups, w.groups, w.reduce_bucket_size)
    reps = [rng.standard_normal(2278).astype(F) for _ in range(4)]
    whole = reduce_scatter_oracle(plan, 0, reps, False)
    for k in range(4):
        part = np.full(570, np.nan, F)
        for b in range(plan.num_buckets):
            got = reduce_scatter_oracle(plan, 0, reps, False, bucket=b, dst=k)[k]
            wrote = ~np.isnan(got)
            assert np.isnan(part[wrote]).all()      # no element written twice
            part[wrote] = got[wrote]
        assert np.array_equal(part.view(np.uint32), whole[k].view(np.uint32))


def test_windowed_replicas_equal_full_replicas():
    rng = np.random.default_rng(8)
    w = workloads.get("tiny")
    plan = plan_oracle(w.numels, w.param_groups, w.groups, w.reduce_bucket_size)
    reps = [rng.standard_normal(2280).astype(F) for _ in range(4)]
    full = reduce_scatter_oracle(plan, 0, [r[:2278] for r in reps], False)
    for k in range(4):
        win = [r[k * 570:(k + 1) * 570] for r in reps]
        got = reduce_scatter_oracle(plan, 0, win, False, dst=k,
                                    flat_bases=[k * 570] * 4)[k]
        assert np.array_equal(got.view(np.uint32), full[k].view(np.uint32))
