"""Plain, slow CPU oracle for partition-aware ZeRO-1/2 gradient reduction.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the C-ABI library
``libzr.so`` and its Python binding) may import, call, link or execute
anything in this package; only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, tables or
constants with the HIP path: the only thing both sides consume is the seeded
input data produced by ``zero_partition_aware_amd.workloads``.

Every floating-point step here is a separate IEEE binary32 operation done by
numpy on float32 arrays (``fl(.)``), because the pages fix the precision of the
method: fp32 master weights, Adam moments and the contiguous fp32 gradient
buffer.  Python ``int`` arithmetic is used for every offset and size.

Pages cited (a reader has these pages, so each citation names page and section):

* [ZeRO-RS blog] "DeepSpeed ZeRO 通信优化深度解析：用 reduce-scatter 分区感知规约替代
  all-reduce", https://blog.gitcode.com/1c986eff0cf5f4ea70019c2fdf8cc263.html
* [Megatron DP] "Megatron-LM 分布式训练（四）：数据并行 DP 与分布式优化器（ZeRO）",
  https://swordlidev.github.io/blog/megatron-lm-04-data-parallel-zero/
* [Collectives Q&A] "07. 大规模训练时通信瓶颈在哪里？AllReduce、AllGather、ReduceScatter
  有什么区别？", https://model.playoffer.cn/interview-resources/
  distributed-training-frameworks/training-communication-allreduce-allgather-reducescatter
* [Adam] Kingma & Ba, "Adam: A Method for Stochastic Optimization" (ICLR 2015),
  Algorithm 1.

Modules:

* ``plan``   -- flat space, equal padded partitions, param_to_partition_ids,
  grad_start_offset, buckets and merged (dst, bucket_offset, numel) slices,
  built twice (interval arithmetic and a brute-force element map).
* ``ipg``    -- main_grad += widen(bf16 grad), per micro-batch, in order.
* ``reduce`` -- rank-ordered sum of grad / N per partition slice, and the
  all-reduce-average reference computed without any plan.
* ``adam``   -- textbook Adam in fp32 (plus an fp64 twin for sanity).
* ``bf16``   -- round-to-nearest-even fp32 -> bf16 from its definition.
* ``ring``   -- literal ring reduce-scatter / all-gather message passing.
* ``volume`` -- communication-volume and per-card byte accounting.

Parity pins: every function is pinned by ``tests/test_oracle_*.py`` against
hand-derived values, closed forms, invariants, brute force or an independent
library routine; none is "parity unpinned".
"""
