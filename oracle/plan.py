"""Oracle O1: the bucket / partition plan.  TEST INFRASTRUCTURE ONLY.

What is computed (all integers, Python ``int``):

* One flat parameter space per process group g, holding that group's params in
  list order, padded at its end so that it splits into R_g *equal* partitions
  ([ZeRO-RS blog §二]: optimizer state and 16-bit grads are cut into
  data-parallel-degree equal parts; [Megatron DP] "分布式优化器" section: each
  card owns 1/DP).  L_g = ceil(T_g / (R_g*align)) * R_g*align, P_g = L_g / R_g.
  The padding is at the end of the group's space, so it belongs to the last
  partition.
* ``param_to_partition_ids[p]``: every partition index the param's flat range
  touches, and ``grad_start_offset[p][k]``: where partition k's piece starts
  inside param p ([ZeRO-RS blog §三.2], the per-param partition metadata used
  by ``average_tensor``).
* Buckets: params are walked in list (ready) order across all groups; a bucket
  holds at most ``reduce_bucket_size`` elements ([ZeRO-RS blog §五], the
  element cap per reduction; [ZeRO-RS blog §四], the IPG bucket).  A param is
  split at a bucket boundary (reading: the cap is hard).
* Slices: the pieces of every param cut at bucket and partition boundaries,
  labelled (dst rank, bucket offset, numel), with adjacent pieces of one bucket
  that share (group, dst) merged into one ([ZeRO-RS blog §三.2], the
  ("reduce", dst, process_group) grouping and the merge of contiguous pieces).
* Divisor D_g = R_g / sp_g, the data-parallel size over the sequence-parallel
  size ([ZeRO-RS blog §六], mean semantics and sequence parallel).  Expert
  params use the expert-data-parallel group ([ZeRO-RS blog §六], MoE bullet):
  here that is simply a group with its own (R, sp).

Two independent constructions are given: ``plan_oracle`` by interval
arithmetic (usable at full model sizes) and ``plan_bruteforce`` from a
per-element map (small inputs only); the tests require them to agree.
"""

from dataclasses import dataclass, field


@dataclass(frozen=True)
class Slice:
    """One merged slice: elements [bucket_offset, +numel) of bucket ``bucket``
    are elements [flat_offset, +numel) of group ``group``'s flat space and
    land at [part_offset, +numel) of partition ``dst``."""
    bucket: int
    group: int
    dst: int
    bucket_offset: int
    flat_offset: int
    part_offset: int
    numel: int


@dataclass
class GroupInfo:
    world: int          # R_g, replicas reduced together
    sp: int             # sequence-parallel size sp_g
    total: int          # T_g, elements of real params
    padded: int         # L_g
    part_numel: int     # P_g
    divisor: int        # D_g = R_g / sp_g (an integer)


@dataclass
class Plan:
    groups: list
    param_group: list
    param_numel: list
    param_offset: list            # o_p inside its group's flat space
    param_to_partition_ids: list  # list of lists of partition indices
    grad_start_offset: list       # list of dicts {k: offset inside param}
    reduce_bucket_size: int
    num_buckets: int
    slices: list = field(default_factory=list)   # in bucket order (pi order)


def _check_inputs(numels, param_groups, groups, reduce_bucket_size, align):
    if reduce_bucket_size <= 0:
        raise ValueError("reduce_bucket_size must be positive")
    if align <= 0:
        raise ValueError("align must be positive")
    if len(numels) != len(param_groups):
        raise ValueError("numels and param_groups differ in length")
    for world, sp in groups:
        if world <= 0 or sp <= 0 or world % sp != 0:
            raise ValueError("each group needs world > 0, sp > 0, sp | world")
    for n, g in zip(numels, param_groups):
        if n <= 0:
            raise ValueError("every param needs numel > 0")
        if not 0 <= g < len(groups):
            raise ValueError("param group index out of range")


def _groups_and_offsets(numels, param_groups, groups, align):
    totals = [0] * len(groups)
    offsets = []
    for n, g in zip(numels, param_groups):
        offsets.append(totals[g])
        totals[g] += n
    infos = []
    for g, (world, sp) in enumerate(groups):
        unit = world * align
        padded = -(-totals[g] // unit) * unit
        infos.append(GroupInfo(world=world, sp=sp, total=totals[g],
                               padded=padded, part_numel=padded // world,
                               divisor=world // sp))
    return infos, offsets


def plan_oracle(numels, param_groups, groups, reduce_bucket_size, align=1):
    """Interval-arithmetic plan.  ``numels[p]``/``param_groups[p]`` list the
    params in ready order; ``groups[g] = (world, sp)``."""
    _check_inputs(numels, param_groups, groups, reduce_bucket_size, align)
    infos, offsets = _groups_and_offsets(numels, param_groups, groups, align)
    B = reduce_bucket_size

    ids_all, gso_all = [], []
    for p, (n, g) in enumerate(zip(numels, param_groups)):
        P = infos[g].part_numel
        o = offsets[p]
        first, last = o // P, (o + n - 1) // P
        ids = list(range(first, last + 1))
        ids_all.append(ids)
        gso_all.append({k: max(0, k * P - o) for k in ids})

    # Walk params in list order; cut each at bucket and partition boundaries.
    pieces = []
    pi = 0
    for p, (n, g) in enumerate(zip(numels, param_groups)):
        P = infos[g].part_numel
        f, end = offsets[p], offsets[p] + n
        while f < end:
            b = pi // B
            dst = f // P
            room_bucket = (b + 1) * B - pi
            room_part = (dst + 1) * P - f
            take = min(end - f, room_bucket, room_part)
            pieces.append(Slice(b, g, dst, pi - b * B, f, f - dst * P, take))
            pi += take
            f += take
    total_pi = pi

    merged = []
    for s in pieces:
        if merged:
            t = merged[-1]
            if (t.bucket, t.group, t.dst) == (s.bucket, s.group, s.dst):
                assert t.bucket_offset + t.numel == s.bucket_offset
                assert t.flat_offset + t.numel == s.flat_offset
                merged[-1] = Slice(t.bucket, t.group, t.dst, t.bucket_offset,
                                   t.flat_offset, t.part_offset,
                                   t.numel + s.numel)
                continue
        merged.append(s)

    return Plan(groups=infos, param_group=list(param_groups),
                param_numel=list(numels), param_offset=offsets,
                param_to_partition_ids=ids_all, grad_start_offset=gso_all,
                reduce_bucket_size=B, num_buckets=-(-total_pi // B),
                slices=merged)


def plan_bruteforce(numels, param_groups, groups, reduce_bucket_size, align=1):
    """The same plan from a literal per-element map (small inputs only).

    Each element e of param p gets: global position pi (list order across all
    groups), bucket pi // B, flat offset f inside its group, destination
    f // P_g and partition offset f - dst*P_g.  Merged slices are then the
    maximal runs of constant (bucket, group, dst) along pi."""
    _check_inputs(numels, param_groups, groups, reduce_bucket_size, align)
    B = reduce_bucket_size
    # Group sizes from scratch, element by element.
    counts = [0] * len(groups)
    elem = []   # (pi, group, flat)
    pi = 0
    for n, g in zip(numels, param_groups):
        for _ in range(n):
            elem.append((pi, g, counts[g]))
            counts[g] += 1
            pi += 1
    infos = []
    for g, (world, sp) in enumerate(groups):
        padded = counts[g]
        while padded % (world * align) != 0:
            padded += 1
        infos.append(GroupInfo(world, sp, counts[g], padded, padded // world,
                               world // sp))

    ids_all, gso_all, offsets = [], [], []
    start = 0
    for n, g in zip(numels, param_groups):
        P = infos[g].part_numel
        flats = [elem[start + j][2] for j in range(n)]
        offsets.append(flats[0])
        ids, gso = [], {}
        for j, f in enumerate(flats):
            k = f // P
            if k not in gso:
                ids.append(k)
                gso[k] = j
        ids_all.append(ids)
        gso_all.append(gso)
        start += n

    slices = []
    for (pi, g, f) in elem:
        P = infos[g].part_numel
        b, dst = pi // B, f // P
        if slices:
            t = slices[-1]
            if (t.bucket, t.group, t.dst) == (b, g, dst):
                assert t.flat_offset + t.numel == f
                slices[-1] = Slice(t.bucket, t.group, t.dst, t.bucket_offset,
                                   t.flat_offset, t.part_offset, t.numel + 1)
                continue
        slices.append(Slice(b, g, dst, pi - b * B, f, f - dst * P, 1))

    return Plan(groups=infos, param_group=list(param_groups),
                param_numel=list(numels), param_offset=offsets,
                param_to_partition_ids=ids_all, grad_start_offset=gso_all,
                reduce_bucket_size=B, num_buckets=-(-len(elem) // B),
                slices=slices)


def slices_for(plan, group, bucket=-1, dst=-1):
    """The merged slices of ``group`` in ``bucket`` (-1: all) going to ``dst``
    (-1: all), in bucket order."""
    return [s for s in plan.slices
            if s.group == group
            and (bucket < 0 or s.bucket == bucket)
            and (dst < 0 or s.dst == dst)]
