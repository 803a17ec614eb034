"""Oracle for copy_grads_in_partition: the reduced elements of one bucket,
laid out in bucket order, moved into the local partition.  TEST
INFRASTRUCTURE ONLY.

[ZeRO-RS blog §三.3]: once a bucket is reduced, each rank copies the reduced
pieces that belong to its own partition out of the bucket into its contiguous
partition gradient buffer; a merged slice (dst, bucket_offset, numel) of the
bucket lands at the slice's offset inside partition dst ([ZeRO-RS blog
§三.2] for the slices).  Elements of the partition that no slice of this
bucket covers are left as they were (NaN here).

The bucket-layout vector the copy reads is what a reduction over the whole
bucket leaves: element bucket_offset + j of the bucket is the rank-ordered
pre-divided mean of the slice's group at flat offset flat_offset + j
([ZeRO-RS blog §六] mean semantics, as in ``reduce``).
"""

import numpy as np

from .reduce import rank_order_mean, _as_f32


def bucket_layout_mean(plan, bucket, replicas_by_group, is_bf16):
    """The bucket's reduced elements in bucket order (float32, NaN where the
    bucket holds nothing).  ``replicas_by_group[g]`` lists group g's replica
    vectors over its whole flat space."""
    n = max((s.bucket_offset + s.numel for s in plan.slices if s.bucket == bucket), default=0)
    out = np.full(n, np.nan, dtype=np.float32)
    for s in plan.slices:
        if s.bucket != bucket:
            continue
        info = plan.groups[s.group]
        xs = [_as_f32(x, is_bf16)[s.flat_offset: s.flat_offset + s.numel]
              for x in replicas_by_group[s.group]]
        out[s.bucket_offset: s.bucket_offset + s.numel] = rank_order_mean(xs, info.divisor)
    return out


def copy_grads_in_partition_oracle(plan, group, bucket, dst, bucket_layout_src):
    """Partition ``dst`` of ``group`` (P_g float32 elements, NaN where this
    bucket has no slice for it) after copying the bucket's slices into it."""
    P = plan.groups[group].part_numel
    src = np.asarray(bucket_layout_src, dtype=np.float32)
    out = np.full(P, np.nan, dtype=np.float32)
    for s in plan.slices:
        if s.group == group and s.bucket == bucket and s.dst == dst:
            out[s.part_offset: s.part_offset + s.numel] = \
                src[s.bucket_offset: s.bucket_offset + s.numel]
    return out
