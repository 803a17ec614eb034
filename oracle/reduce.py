"""Oracles O3/O4: partition-aware pre-divide reduce-scatter, and the plain
all-reduce average it must agree with.  TEST INFRASTRUCTURE ONLY.

Definitions followed:

* Reduce-scatter: GPU i ends with the sum over all GPUs of segment i
  ([Collectives Q&A] "三种集合通信原语", the ReduceScatter definition).
* All-reduce: every GPU ends with the element-wise sum of every GPU's vector
  ([Collectives Q&A], AllReduce definition); all-reduce = reduce-scatter
  followed by all-gather ([ZeRO-RS blog §二]; [Collectives Q&A]
  "Ring-AllReduce = ReduceScatter + AllGather").
* Mean semantics: each gradient is divided by dp_world_size /
  sequence_parallel_size *before* it is sent, so that the result is the
  average over the data-parallel replicas ([ZeRO-RS blog §六]); Megatron
  scales the bucket by 1/DP for the same purpose ([Megatron DP] step 4).
* Each merged slice goes only to its destination partition ([ZeRO-RS blog
  §三.2]) and lands at its partition offset, the ``copy_grads_in_partition``
  step ([ZeRO-RS blog §三.3]).

Arithmetic (the readings of the method that the kernels must reproduce
bit-for-bit): every operation is one fp32 operation; each replica's value is
divided by D first (true IEEE division), then the quotients are summed in rank
order 0, 1, ..., R-1 with the accumulator starting from the rank-0 quotient.
bf16 inputs are widened exactly before anything else.
"""

import numpy as np

from .ipg import widen_bf16


def _as_f32(x, is_bf16):
    return widen_bf16(x) if is_bf16 else np.asarray(x, dtype=np.float32)


def rank_order_mean(values, divisor):
    """fl(...fl(fl(x0/D) + fl(x1/D)) ... + fl(x_{R-1}/D)) element-wise.

    ``values`` is a list of R float32 arrays of one shape, in rank order."""
    d = np.float32(divisor)
    acc = np.divide(values[0], d, dtype=np.float32)
    for x in values[1:]:
        q = np.divide(x, d, dtype=np.float32)
        acc = np.add(acc, q, dtype=np.float32)
    return acc


def reduce_scatter_oracle(plan, group, replicas, is_bf16, bucket=-1, dst=-1,
                          flat_bases=None):
    """Run the merged slices of ``group`` (optionally one bucket / one dst).

    ``replicas[r]`` holds replica r's gradients for flat elements
    [flat_bases[r], flat_bases[r] + len) of the group (full flat space when
    ``flat_bases`` is None).  Returns {dst: float32 partition of P_g elements}
    with NaN marking elements no slice of this call wrote, except that the
    padding (flat elements [T_g, L_g), at the end of the group's space, so in
    the last partition(s)) is 0 when the call covers the last bucket: padding
    is part of no bucket and holds zero gradient."""
    info = plan.groups[group]
    R, P, D = info.world, info.part_numel, info.divisor
    assert len(replicas) == R
    if flat_bases is None:
        flat_bases = [0] * R
    xs = [_as_f32(x, is_bf16) for x in replicas]
    dsts = range(R) if dst < 0 else [dst]
    out = {k: np.full(P, np.nan, dtype=np.float32) for k in dsts}
    for s in plan.slices:
        if s.group != group or (bucket >= 0 and s.bucket != bucket):
            continue
        if s.dst not in out:
            continue
        vals = []
        for r in range(R):
            lo = s.flat_offset - flat_bases[r]
            assert 0 <= lo and lo + s.numel <= xs[r].shape[0], "window miss"
            vals.append(xs[r][lo: lo + s.numel])
        out[s.dst][s.part_offset: s.part_offset + s.numel] = \
            rank_order_mean(vals, D)
    if bucket < 0 or bucket == plan.num_buckets - 1:
        for k in out:
            first_pad = min(P, max(0, info.total - k * P))
            out[k][first_pad:] = 0.0
    return out


def allreduce_average_oracle(replicas, divisor, is_bf16):
    """All-reduce average of full flat vectors, computed with no plan at all:
    every GPU would hold this whole vector."""
    xs = [_as_f32(x, is_bf16) for x in replicas]
    return rank_order_mean(xs, divisor)
