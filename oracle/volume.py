"""Oracle O8: communication-volume and per-card memory accounting.
TEST INFRASTRUCTURE ONLY.

Closed forms the pages state:

* Ring all-reduce moves 2(N-1)/N of the message per card ([Megatron DP]
  "深入：all-reduce 底层算法（NCCL）"; [Collectives Q&A] "三种集合通信原语").
  Reduce-scatter is its first half and all-gather its second half, so each is
  (N-1)/N ([Collectives Q&A] "Ring-AllReduce = ReduceScatter + AllGather").
* busbw = algbw * 2(N-1)/N for an all-reduce ([Megatron DP], same section).
* Mixed-precision Adam holds 16 bytes per parameter: bf16 weight 2, bf16 grad
  2, fp32 master 4, m 4, v 4 ([Megatron DP] "朴素 DP 的致命浪费").
* Per-card bytes for plain DP / ZeRO-1 / ZeRO-1.5 / ZeRO-3: 16, 2+2+12/N,
  2+2/N+12/N, 16/N ([Megatron DP] "ZeRO 各档" table).

Reading used to reconcile the volume claims (the pages disagree on wording;
this counting makes all of them true at once), in units of psi*(N-1)/N with
psi the parameter count:

* plain DP: gradient all-reduce = 2;
* first ZeRO-1 (global all-reduce of grads, then all-gather of the updated
  params): 2 + 1 = 3, i.e. 1.5x DP ([ZeRO-RS blog §一]);
* partition-aware ZeRO-1/2: reduce-scatter + all-gather = 1 + 1 = 2, i.e.
  1.0x DP ([ZeRO-RS blog §一]; [Megatron DP] "通信模式");
* gradient synchronisation alone: reduce-scatter 1 vs all-reduce 2, the
  "half" of [Collectives Q&A] and the "up to 2x" time of [ZeRO-RS blog §一].
"""

from fractions import Fraction


def ring_traffic_per_card(kind, n_cards, message_elems):
    """Exact elements each card sends for one collective over a ring."""
    base = Fraction(n_cards - 1, n_cards) * message_elems
    return {"reduce_scatter": base, "all_gather": base,
            "all_reduce": 2 * base}[kind]


def busbw_factor_allreduce(n_cards):
    return Fraction(2 * (n_cards - 1), n_cards)


def step_volume_units(scheme):
    """Per-step communication in units of psi*(N-1)/N."""
    return {"dp_allreduce": 2,
            "zero1_global_allreduce_then_allgather": 3,
            "zero_partition_aware": 2,
            "grad_sync_reduce_scatter": 1,
            "grad_sync_allreduce": 2}[scheme]


def adam_bytes_per_param():
    parts = {"bf16_weight": 2, "bf16_grad": 2, "fp32_master": 4,
             "adam_m": 4, "adam_v": 4}
    return sum(parts.values()), parts


def per_card_bytes_per_param(scheme, n):
    """Per-card bytes per parameter for the ZeRO table's rows."""
    n = Fraction(n)
    return {"dp": Fraction(16),
            "zero1": 2 + 2 + 12 / n,
            "zero1.5": 2 + 2 / n + 12 / n,
            "zero3": 16 / n}[scheme]
