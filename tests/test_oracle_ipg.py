"""Pins for oracle O2 (IPG accumulation into the fp32 main_grad window)."""

import numpy as np

from oracle.ipg import ipg_accumulate_oracle
from zero_partition_aware_amd import workloads

F = np.float32


def _bf16_of_ints(v):
    # Integers with |v| <= 256 are exact in bf16: their fp32 pattern has a zero
    # low half, so the bf16 pattern is the high half.
    return (np.asarray(v, F).view(np.uint32) >> 16).astype(np.uint16)


def test_integer_bf16_sums_exact_with_window_clipping():
    rng = np.random.default_rng(0)
    numels = [5, 17, 1, 40, 9]
    offsets = [0, 5, 22, 23, 63]
    total = 72
    mbs = 4
    grads = [[rng.integers(-256, 257, size=n) for n in numels] for _ in range(mbs)]
    for base, length in [(0, 72), (10, 30), (22, 1), (60, 12), (0, 5)]:
        mg = np.zeros(length, F)
        for mb in range(mbs):
            ipg_accumulate_oracle(mg, base, offsets, list(range(5)),
                                  [_bf16_of_ints(g) for g in grads[mb]], True)
        want = [0] * total
        for mb in range(mbs):
            for p in range(5):
                for j in range(numels[p]):
                    want[offsets[p] + j] += int(grads[mb][p][j])
        assert mg.tolist() == [float(x) for x in want[base:base + length]]


def test_micro_batch_order_is_call_order():
    # fl(fl(fl(0 + 2^24) + 1) + 1) - 2^24 = 0 in call order; 2 in reverse.
    seq = [2.0 ** 24, 1.0, 1.0, -(2.0 ** 24)]
    for order, want in [(seq, 0.0), (seq[::-1], 2.0)]:
        mg = np.zeros(1, F)
        for v in order:
            ipg_accumulate_oracle(mg, 0, [0], [0], [np.array([v], F)], False)
        assert mg[0] == want


def test_params_outside_window_are_skipped():
    mg = np.zeros(4, F)
    ipg_accumulate_oracle(mg, 100, [0, 104], [0, 1],
                          [np.ones(10, F), np.ones(3, F)], False)
    assert mg.tolist() == [0.0] * 4


def test_random_bf16_is_deterministic_elementwise():
    g = workloads.host_bf16_normal(17, 1000, 1e-3)
    a = np.zeros(1000, F)
    b = np.zeros(1000, F)
    ipg_accumulate_oracle(a, 0, [0], [0], [g], True)
    for i in range(1000):
        ipg_accumulate_oracle(b[i:i + 1], i, [0], [0], [g], True)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
