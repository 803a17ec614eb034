"""Pins for oracles O7/O8: ring message passing and the volume accounting."""

from fractions import Fraction

import numpy as np
import pytest

from oracle.reduce import rank_order_mean
from oracle.ring import (ring_all_gather_oracle, ring_order_sum,
                         ring_reduce_scatter_oracle)
from oracle.volume import (adam_bytes_per_param, busbw_factor_allreduce,
                           per_card_bytes_per_param, ring_traffic_per_card,
                           step_volume_units)

F = np.float32


@pytest.mark.parametrize("N", [1, 2, 3, 5, 8])
def test_ring_rs_equals_direct_sum_on_integers(N):
    rng = np.random.default_rng(N)
    C = 13
    bufs = [rng.integers(-1000, 1000, size=N * C).astype(F) for _ in range(N)]
    out, sent = ring_reduce_scatter_oracle(bufs)
    for k in range(N):
        want = sum(b[k * C:(k + 1) * C].astype(np.int64) for b in bufs)
        assert out[k][k * C:(k + 1) * C].tolist() == want.astype(float).tolist()
    assert sent == [(N - 1) * C] * N
    assert all(Fraction(s) == ring_traffic_per_card("reduce_scatter", N, N * C)
               for s in sent)


def test_ring_rs_floats_follow_ring_order():
    rng = np.random.default_rng(0)
    N, C = 8, 4096
    bufs = [rng.standard_normal(N * C).astype(F) for _ in range(N)]
    out, _ = ring_reduce_scatter_oracle(bufs)
    differs = 0
    for k in range(N):
        got = out[k][k * C:(k + 1) * C]
        assert np.array_equal(got.view(np.uint32),
                              ring_order_sum(bufs, k).view(np.uint32))
        rank_order = rank_order_mean([b[k * C:(k + 1) * C] for b in bufs], 1)
        differs += int((got != rank_order).sum())
        # Both orders are within the usual bound of the exact sum.
        exact = sum(b[k * C:(k + 1) * C].astype(np.float64) for b in bufs)
        absum = sum(np.abs(b[k * C:(k + 1) * C].astype(np.float64)) for b in bufs)
        gamma = (N - 1) * 2.0 ** -24 / (1 - (N - 1) * 2.0 ** -24)
        assert np.all(np.abs(got - exact) <= gamma * absum)
    assert differs > 0   # the summation orders really are different


def test_partial_steps_schedule():
    # After step s (0-based) card k has just summed chunk (k - s - 2) mod N.
    N, C = 4, 1
    bufs = [np.array([10.0 ** r] * N, F) for r in range(N)]   # card r holds 10^r
    out, _ = ring_reduce_scatter_oracle(bufs, steps=1)
    for k in range(N):
        c = (k - 2) % N
        assert out[k][c] == F(10.0 ** k + 10.0 ** ((k - 1) % N))


@pytest.mark.parametrize("N", [2, 4, 8])
def test_rs_then_ag_is_allreduce(N):
    rng = np.random.default_rng(N + 100)
    C = 7
    bufs = [rng.integers(-50, 50, size=N * C).astype(F) for _ in range(N)]
    rs, sent_rs = ring_reduce_scatter_oracle(bufs)
    ag, sent_ag = ring_all_gather_oracle(rs)
    total = sum(b.astype(np.int64) for b in bufs).astype(float).tolist()
    for k in range(N):
        assert ag[k].tolist() == total
    per_card = [a + b for a, b in zip(sent_rs, sent_ag)]
    assert all(Fraction(s) == ring_traffic_per_card("all_reduce", N, N * C)
               for s in per_card)
    assert busbw_factor_allreduce(N) == Fraction(2 * (N - 1), N)


def test_volume_ratios():
    dp = step_volume_units("dp_allreduce")
    assert Fraction(step_volume_units("zero1_global_allreduce_then_allgather"), dp) == Fraction(3, 2)
    assert Fraction(step_volume_units("zero_partition_aware"), dp) == 1
    assert Fraction(step_volume_units("grad_sync_allreduce"),
                    step_volume_units("grad_sync_reduce_scatter")) == 2
    for N in (2, 8, 64):
        assert ring_traffic_per_card("all_reduce", N, 1) == \
            ring_traffic_per_card("reduce_scatter", N, 1) + ring_traffic_per_card("all_gather", N, 1)


def test_byte_table():
    total, parts = adam_bytes_per_param()
    assert total == 16 and parts["fp32_master"] + parts["adam_m"] + parts["adam_v"] == 12
    assert per_card_bytes_per_param("zero1", 1) == per_card_bytes_per_param("dp", 1) == 16
    assert per_card_bytes_per_param("zero3", 8) == 2
    assert per_card_bytes_per_param("zero1", 8) == Fraction(11, 2)
    assert per_card_bytes_per_param("zero1.5", 8) == Fraction(2) + Fraction(14, 8)


def test_all_gather_is_concatenation_by_brute_force():
    from oracle.allgather import all_gather_oracle, all_gather_window_oracle
    rng = np.random.default_rng(3)
    for R, P, T in [(4, 5, 18), (2, 3, 6), (8, 1, 5), (3, 7, 21)]:
        parts = [rng.standard_normal(P).astype(F) for _ in range(R)]
        full = all_gather_oracle(parts, T)
        for f in range(T):                       # element f lives in partition f // P
            assert full[f] == parts[f // P][f % P]
        assert full.shape[0] == T
        got = all_gather_window_oracle(parts, T, 2, 100)
        assert np.array_equal(got, full[2:])


def test_reduce_scatter_then_all_gather_is_all_reduce():
    # All-reduce = reduce-scatter followed by all-gather: gathering the
    # shards of the partition-aware reduction gives the all-reduce average.
    from oracle.allgather import all_gather_oracle
    from oracle.plan import plan_oracle
    from oracle.reduce import allreduce_average_oracle, reduce_scatter_oracle
    rng = np.random.default_rng(4)
    numels = [37, 2112, 129]
    plan = plan_oracle(numels, [0, 0, 0], [(4, 1)], 1000)
    reps = [rng.standard_normal(2278).astype(F) for _ in range(4)]
    shards = reduce_scatter_oracle(plan, 0, reps, False)
    full = all_gather_oracle([shards[k] for k in range(4)], 2278)
    ar = allreduce_average_oracle(reps, 4, False)
    assert np.array_equal(full.view(np.uint32), ar.view(np.uint32))


@pytest.mark.parametrize("N", [2, 4, 8])
def test_step_volume_units_match_simulated_ring_traffic(N):
    """Each scheme's per-step volume, in units of psi*(N-1)/N, equals what the
    literal ring simulation sends per card for the collectives the scheme runs
    (gradient all-reduce = reduce-scatter + all-gather; parameter all-gather)."""
    C = 5
    M = N * C
    unit = Fraction(N - 1, N) * M
    bufs = [np.ones(M, F) for _ in range(N)]
    rs_out, rs = ring_reduce_scatter_oracle(bufs)
    _, ag = ring_all_gather_oracle(rs_out)
    rs, ag = Fraction(rs[0]), Fraction(ag[0])
    assert all(Fraction(x) == rs for x in ring_reduce_scatter_oracle(bufs)[1])
    simulated = {"dp_allreduce": rs + ag,
                 "zero1_global_allreduce_then_allgather": rs + ag + ag,
                 "zero_partition_aware": rs + ag,
                 "grad_sync_reduce_scatter": rs,
                 "grad_sync_allreduce": rs + ag}
    for scheme, sent in simulated.items():
        assert step_volume_units(scheme) * unit == sent, scheme
