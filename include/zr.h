/*
 * zr.h -- C ABI of libzr: partition-aware ZeRO-1/2 gradient reduction and
 * partition Adam on one MI355X (gfx950).
 *
 * Pages cited (each citation names the page and the section on it):
 *   [ZeRO-RS blog]  "DeepSpeed ZeRO 通信优化深度解析：用 reduce-scatter 分区感知规约替代
 *                   all-reduce", https://blog.gitcode.com/1c986eff0cf5f4ea70019c2fdf8cc263.html
 *   [Megatron DP]   "Megatron-LM 分布式训练（四）：数据并行 DP 与分布式优化器（ZeRO）",
 *                   https://swordlidev.github.io/blog/megatron-lm-04-data-parallel-zero/
 *   [Collectives]   "07. 大规模训练时通信瓶颈在哪里？AllReduce、AllGather、ReduceScatter
 *                   有什么区别？", model.playoffer.cn interview resources
 *   [Adam]          Kingma & Ba, "Adam: A Method for Stochastic Optimization",
 *                   Algorithm 1.
 *
 * What the library computes.  N data-parallel replicas each hold a gradient
 * for the same flat parameter space.  Instead of an all-reduce, every
 * replica k only needs the average gradient of the partition it owns
 * (reduce-scatter), then applies Adam to its own fp32 master partition.  Here
 * the N replicas' gradient buffers are resident in one GPU's HBM, so the
 * "reduce-scatter" is a local streaming kernel that reads the N replica
 * windows of a partition and writes that partition.
 *
 * Conventions for every call:
 *   - Device memory is owned by the caller (e.g. torch tensors passed as raw
 *     device pointers).  The library never frees or reallocates it.
 *     Pointers need only be element-aligned.  The fastest path needs the
 *     streams of a segment to share one 4-element phase (16-byte accesses
 *     for fp32, 8-byte for bf16); otherwise a variant takes the vector path
 *     with streams merely 4-byte aligned (bf16 streams an odd number of
 *     elements apart read with shifted loads), somewhat slower.  Partition sizes that
 *     are a multiple of 4 (align >= 4 in zr_plan_buckets) keep every rank on
 *     the fastest path.  Replica tiles are placed on whole 128-byte lines
 *     whenever the other streams allow it, so buffers whose starts share
 *     their offset within a line stream fastest.
 *   - The library owns a plan (create with zr_plan_buckets, free with
 *     zr_plan_free).  A plan is immutable; small device tables derived from
 *     it are built on first use and freed with it.  The first use of a
 *     (group, bucket range, dst, device) selection allocates its table and
 *     uploads it synchronously (one hipMalloc and one hipMemcpy of 40 bytes
 *     per segment, typically tens of microseconds); later calls reuse it.
 *     A call recorded into a HIP graph must not be the first use of its
 *     selection: make it once outside the capture (or use
 *     zr_reduce_scatter_adam_noalloc, which needs no table).
 *   - Work is enqueued on the caller's HIP stream; nothing synchronises
 *     implicitly.  Completion is the caller's stream synchronisation.  One
 *     call may enqueue several kernel launches: selections whose traffic
 *     exceeds about 2 GiB are cut into equal launches of at most that much
 *     (in one long launch the GPU's XCDs drift apart in the address space,
 *     which costs bandwidth; a launch boundary realigns them).  Reduce
 *     launches may reserve LDS they never touch, to hold each CU to a
 *     measured number of their workgroups (zr_reduce_launch_occupancy).
 *   - Every call returns a zr_status.  Arguments are validated before any
 *     work is enqueued; on failure no output is touched and zr_last_error()
 *     returns a message (thread-local).  No C++ exception crosses the ABI.
 *   - Arithmetic is IEEE binary32 without FMA contraction, with subnormals
 *     kept; NaN and Inf propagate and are not detected.
 */
#ifndef ZR_H
#define ZR_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ZR_VERSION 100   /* 1.0.0 */
#define ZR_MAX_WORLD 64  /* largest replica count one reduction accepts */

typedef enum {
  ZR_OK = 0,
  ZR_ERR_INVALID = 1,      /* bad argument; nothing enqueued */
  ZR_ERR_OOM = 2,          /* host or device allocation failed */
  ZR_ERR_HIP = 3,          /* a HIP runtime call or launch failed */
  ZR_ERR_UNSUPPORTED = 4   /* valid request this library does not implement */
} zr_status;

typedef enum { ZR_FP32 = 0, ZR_BF16 = 1 } zr_dtype;

/* One parameter, in list (gradient-ready) order.  numel > 0; group indexes
 * the zr_group array. */
typedef struct { int64_t numel; int32_t group; } zr_param;

/* A reduction group: world = R_g replicas reduced together (the data-parallel
 * group, or the expert-data-parallel group for MoE expert params,
 * [ZeRO-RS blog §六] MoE bullet); sp = sequence_parallel_size.  The
 * pre-divide divisor is D_g = world / sp ([ZeRO-RS blog §六] mean
 * semantics); sp must divide world. */
typedef struct { int32_t world; int32_t sp; } zr_group;

/* One merged slice: elements [bucket_offset, +numel) of bucket `bucket` are
 * flat elements [flat_offset, +numel) of group `group` and belong to
 * partition `dst` at [part_offset, +numel) ([ZeRO-RS blog §三.2]: slices
 * (dst_rank, bucket_offset, numel), contiguous pieces with one destination
 * merged). */
typedef struct {
  int64_t bucket;
  int32_t group;
  int32_t dst;
  int64_t bucket_offset;
  int64_t flat_offset;
  int64_t part_offset;
  int64_t numel;
} zr_slice;

/* Replica r's gradients for flat elements [flat_base, flat_base + len) of a
 * group: either the whole flat space (flat_base 0) or just the window a
 * partition needs.  Element type is given by the call's zr_dtype. */
typedef struct { const void* ptr; int64_t flat_base; int64_t len; } zr_replica;

/* Adam hyper-parameters ([Adam] Algorithm 1; no weight decay).  The derived
 * fp32 constants b1, 1-b1, b2, 1-b2, 1-b1^step, 1-b2^step, lr and eps are each
 * formed in double and rounded once to fp32.  step >= 1. */
typedef struct { double lr, beta1, beta2, eps; int64_t step; } zr_adam;

typedef struct zr_plan zr_plan;

/* ------------------------------------------------------------- planning --- */

/* zr_plan_buckets -- build the bucket/partition plan.
 * [ZeRO-RS blog §二] (equal data-parallel partitions), §三.2
 * (param_to_partition_ids, grad_start_offset, slicing by destination and
 * merging), §四 (IPG bucket filled in ready order), §五 (reduce_bucket_size is
 * an element cap); [Megatron DP] "梯度缓冲区+分桶+overlap" (contiguous buffer
 * split into buckets).
 *   params[n_params]      params in list order (read only, not retained).
 *   groups[n_groups]      reduction groups (read only, not retained).
 *   reduce_bucket_size    B > 0, elements per bucket; buckets run over the
 *                         whole list in order and split params at their
 *                         boundaries (the cap is hard).
 *   partition_gradients   0 = ZeRO-1, 1 = ZeRO-2 (recorded; it changes no
 *                         number: the library never touches non-local
 *                         regions in either stage).
 *   align                 >= 1: each group's flat space is padded at its end
 *                         to a multiple of world*align, so that every
 *                         partition size P_g is a multiple of align.
 *   out                   receives the new plan (owned by the caller, free
 *                         with zr_plan_free).
 * Errors: ZR_ERR_INVALID for numel <= 0, world <= 0, sp <= 0, sp not dividing
 * world, world > ZR_MAX_WORLD, B <= 0, align <= 0, a group index out of
 * range, int64 overflow of a padded size, or a null pointer; ZR_ERR_OOM. */
zr_status zr_plan_buckets(const zr_param* params, int64_t n_params,
                          const zr_group* groups, int32_t n_groups,
                          int64_t reduce_bucket_size,
                          int32_t partition_gradients, int64_t align,
                          zr_plan** out);

/* Frees the plan and its device launch tables.  Freeing device memory waits
 * for the device's outstanding work (as hipFree does), so a plan may be freed
 * while kernels that use it are still queued; it must not be used again. */
void zr_plan_free(zr_plan* plan);

/* Plan queries.  Each reads the plan only; ZR_ERR_INVALID for a null plan or
 * output pointer or an index out of range.
 *
 * Number of buckets: the list's elements in order, cut every
 * reduce_bucket_size elements ([ZeRO-RS blog §五] reduce_bucket_size; §四 the
 * IPG bucket the gradients fill). */
zr_status zr_plan_num_buckets(const zr_plan* plan, int64_t* out);
/* Number of params in the list the plan was built from. */
zr_status zr_plan_num_params(const zr_plan* plan, int64_t* out);
/* The recorded stage flag, 0 = ZeRO-1, 1 = ZeRO-2 ([ZeRO-RS blog §三.1]
 * partition_gradients). */
zr_status zr_plan_partition_gradients(const zr_plan* plan, int32_t* out);

/* Group g's sizes: total T_g, padded L_g, partition P_g = L_g / R_g, and the
 * divisor D_g = R_g / sp_g as a float ([ZeRO-RS blog §二] equal partitions of
 * the padded flat space; §六 the mean over dp_world_size / sp_size, and the
 * expert-parallel group reduced over its own ranks).  Any output pointer may
 * be null. */
zr_status zr_plan_group_info(const zr_plan* plan, int32_t g, int64_t* total,
                             int64_t* padded, int64_t* part_numel,
                             float* divisor);

/* Offset o_p of param p inside its group's flat space: the params of a group
 * laid end to end in list order ([ZeRO-RS blog §二] the flattened parameter
 * space; [Megatron DP] "梯度缓冲区+分桶+overlap" one contiguous buffer). */
zr_status zr_plan_param_offset(const zr_plan* plan, int64_t p, int64_t* out);

/* param_to_partition_ids[p] ([ZeRO-RS blog §三.2]): the partitions the param
 * touches, ascending.  *ids points into the plan (valid until zr_plan_free). */
zr_status zr_plan_param_partitions(const zr_plan* plan, int64_t p,
                                   const int32_t** ids, int32_t* n);

/* grad_start_offset for (p, k) ([ZeRO-RS blog §三.2]): where partition k's
 * piece starts inside param p, max(0, k*P_g - o_p).  ZR_ERR_INVALID when the
 * param does not touch partition k. */
zr_status zr_plan_grad_start_offset(const zr_plan* plan, int64_t p, int32_t k,
                                    int64_t* out);

/* The buckets param p feeds: [*first, *last] (a param split at a bucket
 * border feeds several).  A bucket is complete once every param feeding it
 * has been accumulated -- the trigger of its reduction ([ZeRO-RS blog] §四:
 * a full bucket starts average_tensor). */
zr_status zr_plan_param_buckets(const zr_plan* plan, int64_t p, int64_t* first,
                                int64_t* last);

/* The merged slices of one bucket (bucket >= 0) or of all buckets
 * (bucket == -1), in bucket order: each piece of a param inside a bucket,
 * cut at partition borders, tagged with its destination rank, and adjacent
 * pieces with the same (group, destination) merged ([ZeRO-RS blog §三.2] the
 * slicing and merging of average_tensor).  *s points into the plan. */
zr_status zr_plan_slices(const zr_plan* plan, int64_t bucket,
                         const zr_slice** s, int64_t* n);

/* The launch shape of a reduce call, without making it (host only; no GPU
 * needed): the tiles of the selection -- `group`, the buckets [bucket_first,
 * bucket_first + bucket_count), destination `dst` (-1 = every destination)
 * -- and the kernel launches zr_reduce_scatter_local_range (fused = 0) or
 * zr_reduce_scatter_adam_range (fused = 1, with_grad_out = whether grad_out
 * is given) cut it into, for grad_dtype replicas.  The same selection
 * through the one-bucket calls has the same shape.  A call over a selection
 * that moves more than about 2 GiB makes several equal launches on its
 * stream; a capped call makes as many.  *tiles and *launches are 0 for a
 * selection with no slices.  Either output pointer may be null, not both.
 * Errors: ZR_ERR_INVALID for a bad group, range, dst or dtype.
 * ([ZeRO-RS blog §三.2]: the selection is the merged slices of the bucket
 * range bound for `dst`.) */
zr_status zr_plan_reduce_launches(const zr_plan* plan, int32_t group,
                                  int64_t bucket_first, int64_t bucket_count,
                                  int32_t dst, zr_dtype grad_dtype, int32_t fused,
                                  int32_t with_grad_out, int64_t* tiles,
                                  int64_t* launches);

/* How an uncapped reduce call shares the chip (host only; no GPU needed),
 * for `world` replicas of grad_dtype through zr_reduce_scatter_local and its
 * range form (fused = 0) or zr_reduce_scatter_adam and its range and
 * no-allocation forms (fused = 1).  *wgs_per_cu: how many of the call's
 * workgroups one CU may hold at once; 0 = as many as the kernel's registers
 * allow, otherwise each launch reserves LDS it never touches, so that no
 * more fit.  *weighted: 1 when each launch gives the odd-numbered XCDs 31/32
 * of the tiles the even-numbered ones take, 0 for equal shares.  Grid-capped
 * calls (zr_reduce_scatter_adam_capped) reserve no LDS and take equal shares
 * whatever this says.  Neither changes any result; both matter to a caller
 * that runs the reduction beside other work on the GPU, as the method does
 * when it overlaps the reduction with the backward ([ZeRO-RS blog §四]:
 * overlap_comm).  Either output pointer may be null, not both.
 * Errors: ZR_ERR_INVALID for world < 1 or an unsupported dtype. */
zr_status zr_reduce_launch_occupancy(zr_dtype grad_dtype, int32_t fused, int32_t world,
                                     int32_t* wgs_per_cu, int32_t* weighted);

/* ------------------------------------------------------------- kernels --- */

/* zr_ipg_accumulate -- add each listed param's gradient into the contiguous
 * fp32 gradient buffer ([Megatron DP] "深入：朴素 DP 的 all-reduce" step 2:
 * main_grad.add_(grad) into an fp32 buffer; [ZeRO-RS blog §四] IPG bucket).
 *   param_ids[n], grads[n]  host arrays: grads[i] is a device pointer to
 *                           param param_ids[i]'s numel gradient elements of
 *                           type grad_dtype.  All params must be in one group.
 *   main_grad               device fp32 window holding flat elements
 *                           [window_base, window_base + window_len) of that
 *                           group; each param is clipped to the window.
 * Per element: main_grad[f - window_base] = fl(main_grad + widen(grad)).
 * Repeated calls (micro-batches) accumulate in call order.  The caller zeroes
 * main_grad at the start of a step.  Params listed twice in one call are
 * rejected (ZR_ERR_INVALID) because their adds would race. */
zr_status zr_ipg_accumulate(const zr_plan* plan, const int64_t* param_ids,
                            const void* const* grads, int64_t n,
                            zr_dtype grad_dtype, float* main_grad,
                            int64_t window_base, int64_t window_len,
                            hipStream_t stream);

/* zr_ipg_accumulate_first -- the first micro-batch of a step: what
 * zr_ipg_accumulate gives on a main_grad window zeroed at the start of the
 * step, without the zeroing and without reading main_grad ([Megatron DP]
 * "深入：朴素 DP 的 all-reduce" step 2: the fp32 buffer is zeroed each step
 * and each micro-batch's gradient is added into it).  Same arguments and
 * errors as zr_ipg_accumulate.  Per element of each listed param (clipped to
 * the window): main_grad[f - window_base] = fl(+0 + widen(grad)), the bits
 * the add into +0 gives (a -0 gradient gives +0).  Elements of the window no
 * listed param covers are not written.  Later micro-batches use
 * zr_ipg_accumulate.  It moves s + 4 bytes per element instead of s + 8. */
zr_status zr_ipg_accumulate_first(const zr_plan* plan, const int64_t* param_ids,
                                  const void* const* grads, int64_t n,
                                  zr_dtype grad_dtype, float* main_grad,
                                  int64_t window_base, int64_t window_len,
                                  hipStream_t stream);

/* zr_reduce_scatter_local -- the partition-aware reduction with its copy
 * into the local partition ([ZeRO-RS blog §三.2, §三.3, §六];
 * [Megatron DP] step 4; [Collectives] ReduceScatter definition).
 * For every merged slice of `group` in `bucket` (-1 = all buckets) whose
 * destination is `dst` (-1 = every destination):
 *   part[dst][part_offset + j] =
 *     fl(...fl(fl(x_0/D) + fl(x_1/D)) ... + fl(x_{R-1}/D)),
 *   x_r = replica r's element at flat offset flat_offset + j,
 * summed in rank order 0..R-1 in fp32 (bf16 inputs widened exactly), with a
 * true IEEE division by D_g.  When the call covers the last bucket it also
 * writes 0 to the padding (flat [T_g, L_g)) of the selected partitions.
 *   reps[R_g]      replica windows (host array); each must cover every slice
 *                  the call reads, else ZR_ERR_INVALID.
 *   part_out       host array of device fp32 partition pointers (P_g
 *                  elements each): R_g entries indexed by destination when
 *                  dst == -1, else one entry for partition dst.
 * Partition elements outside the selected slices are not touched. */
zr_status zr_reduce_scatter_local(const zr_plan* plan, int32_t group,
                                  int64_t bucket, int32_t dst,
                                  const zr_replica* reps, zr_dtype grad_dtype,
                                  float* const* part_out, hipStream_t stream);

/* zr_reduce_scatter_local_range -- zr_reduce_scatter_local over the buckets
 * [bucket_first, bucket_first + bucket_count) in one call: every bucket
 * completed since the last call reduced together ([ZeRO-RS blog §四]: each
 * IPG bucket is reduced once it is full; [Megatron DP]
 * "梯度缓冲区+分桶+overlap": a bucket's gradient sync starts once all its
 * grads are ready).  Results are bit-identical to one zr_reduce_scatter_local
 * call per bucket; the range is carried by one launch table (built on its
 * first use, like any selection's) and as few launches as its traffic allows,
 * instead of one launch per bucket.  bucket_count == 0 enqueues nothing;
 * ZR_ERR_INVALID when bucket_first < 0, bucket_count < 0 or the range runs
 * past the last bucket.  Padding is written when the range covers the last
 * bucket. */
zr_status zr_reduce_scatter_local_range(const zr_plan* plan, int32_t group,
                                        int64_t bucket_first, int64_t bucket_count,
                                        int32_t dst, const zr_replica* reps,
                                        zr_dtype grad_dtype, float* const* part_out,
                                        hipStream_t stream);

/* zr_copy_grads_in_partition -- the standalone copy of already reduced slices
 * into the local contiguous partition buffer ([ZeRO-RS blog §三.3]):
 *   part_out[part_offset + j] = bucket_layout_src[bucket_offset + j]
 * for every slice of `group` in bucket `bucket` (>= 0) with destination
 * `dst` (>= 0).  bucket_layout_src holds that bucket's reduced elements in
 * bucket order (fp32). */
zr_status zr_copy_grads_in_partition(const zr_plan* plan, int32_t group,
                                     int64_t bucket, int32_t dst,
                                     const float* bucket_layout_src,
                                     float* part_out, hipStream_t stream);

/* zr_adam_partition -- Adam on one partition's fp32 master, m and v
 * ([Megatron DP] "通信模式": each card updates its own 1/DP slice with its
 * fp32 master; [Adam] Algorithm 1), in fp32 per element:
 *   m' = b1*m + (1-b1)*g;  v' = b2*v + (1-b2)*(g*g)
 *   theta' = theta - (lr*(m'/(1-b1^t))) / (sqrt(v'/(1-b2^t)) + eps)
 * then param_bf16 = round-to-nearest-even(theta') when param_bf16 is not
 * null (NaN stays a quiet NaN).  master, m, v updated in place; n >= 0. */
zr_status zr_adam_partition(const zr_adam* h, const float* grad, float* master,
                            float* m, float* v, uint16_t* param_bf16,
                            int64_t n, hipStream_t stream);

/* zr_reduce_scatter_adam -- zr_reduce_scatter_local for one destination
 * fused with zr_adam_partition on that partition: each reduced element stays
 * in a register and feeds Adam.  Bit-identical to the two calls in sequence.
 * Only the elements of the selected slices (plus the padding when the call
 * covers the last bucket, updated with a zero gradient) are updated.
 * dst >= 0: master, m, v (and param_bf16, grad_out when not null) are that
 * partition's P_g-element buffers.  dst == -1: every rank's step in one
 * call; the buffers hold all R_g partitions back to back (L_g = R_g*P_g
 * elements, partition d from element d*P_g), i.e. the group's whole padded
 * flat space.  grad_out receives the reduced gradient.  Each partition's
 * result is the same, bit for bit, as its own call with dst = d. */
zr_status zr_reduce_scatter_adam(const zr_plan* plan, int32_t group,
                                 int64_t bucket, int32_t dst,
                                 const zr_replica* reps, zr_dtype grad_dtype,
                                 const zr_adam* h, float* master, float* m,
                                 float* v, uint16_t* param_bf16,
                                 float* grad_out, hipStream_t stream);

/* zr_reduce_scatter_adam_range -- zr_reduce_scatter_adam over the buckets
 * [bucket_first, bucket_first + bucket_count), the fused counterpart of
 * zr_reduce_scatter_local_range (same citations and range rules).
 * Bit-identical to one zr_reduce_scatter_adam call per bucket: Adam updates
 * only the elements of the selected slices (plus the padding when the range
 * covers the last bucket). */
zr_status zr_reduce_scatter_adam_range(const zr_plan* plan, int32_t group,
                                       int64_t bucket_first, int64_t bucket_count,
                                       int32_t dst, const zr_replica* reps,
                                       zr_dtype grad_dtype, const zr_adam* h,
                                       float* master, float* m, float* v,
                                       uint16_t* param_bf16, float* grad_out,
                                       hipStream_t stream);

/* zr_reduce_scatter_adam_capped -- zr_reduce_scatter_adam on launches of at
 * most max_workgroups workgroups each (>= 1; ZR_ERR_INVALID otherwise), each
 * workgroup walking its launch's tiles in steps of the grid (the launches
 * are the uncapped call's, zr_plan_reduce_launches).  For a reduction that
 * overlaps the backward pass on a second stream ([ZeRO-RS blog] §四: each
 * IPG bucket is reduced as soon as it is full, while backward continues;
 * [Megatron DP] "梯度缓冲区+分桶+overlap"): the cap bounds the workgroup
 * slots the reduction holds at once, leaving the rest to the backward's
 * kernels; with one tile in flight per workgroup, the HBM-bound reduction
 * slows as the cap shrinks.  Results are bit-identical to
 * zr_reduce_scatter_adam for every cap (the same per-element code); only the
 * launch shape differs.  Errors as zr_reduce_scatter_adam. */
zr_status zr_reduce_scatter_adam_capped(const zr_plan* plan, int32_t group,
                                        int64_t bucket, int32_t dst,
                                        const zr_replica* reps, zr_dtype grad_dtype,
                                        const zr_adam* h, float* master, float* m,
                                        float* v, uint16_t* param_bf16,
                                        float* grad_out, int32_t max_workgroups,
                                        hipStream_t stream);

/* zr_reduce_scatter_adam_noalloc -- zr_reduce_scatter_adam for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Same arguments, results and
 * errors, bit for bit; it allocates no device memory.  Where
 * zr_reduce_scatter_adam uploads the selection's segment table into memory
 * the library allocates (once per selection), this call stages the table on
 * `stream` before its reduce launches, into a fixed device array of 256 KiB
 * that the library holds on each GPU for the life of the process: at most
 * 6,552 segments per selection, else ZR_ERR_INVALID before anything is
 * enqueued.  (A selection's segments are its merged slices plus one padding
 * segment per selected partition that holds padding.)  Every call on one GPU
 * shares that GPU's array and leaves its own table there, so calls that
 * overlap on one GPU -- on different streams without an ordering between
 * them -- race: order them on one stream or with events.  The plan's
 * host-side segment list for a selection is still built on its first use
 * (host memory). */
zr_status zr_reduce_scatter_adam_noalloc(const zr_plan* plan, int32_t group,
                                         int64_t bucket, int32_t dst,
                                         const zr_replica* reps, zr_dtype grad_dtype,
                                         const zr_adam* h, float* master, float* m,
                                         float* v, uint16_t* param_bf16,
                                         float* grad_out, hipStream_t stream);

/* zr_ring_rs_step -- one step of ring reduce-scatter with every card's buffer
 * resident in this GPU ([Megatron DP] "深入：all-reduce 底层算法（NCCL）", ring
 * reduce-scatter phase).  rank_bufs[n_ranks] (host array of device fp32
 * buffers of n_ranks*chunk_numel elements).  For every rank k:
 *   buf_k[c] = fl(buf_k[c] + buf_{k-1}[c]),  c = (k - step - 2) mod n_ranks,
 * element-wise over the chunk.  After steps 0..n_ranks-2, rank k's chunk k
 * holds the sum over ranks in ring order k+1, ..., k.  0 <= step <= n-2. */
zr_status zr_ring_rs_step(float* const* rank_bufs, int32_t n_ranks,
                          int64_t chunk_numel, int32_t step,
                          hipStream_t stream);

/* zr_all_gather_params -- rebuild the full flat vector of a group from its
 * R_g partitions after the partition update ([Megatron DP] "通信模式": the
 * all-gather that stitches the updated 1/DP slices back into full weights for
 * the next forward; [Collectives] AllGather definition):
 *   out[f - out_base] = parts[f / P_g][f % P_g]
 * for flat f in [out_base, out_base + out_len), which must lie inside the
 * group's real elements [0, T_g) (padding is not a parameter).
 *   parts[R_g]  host array of device partition pointers (P_g elements each;
 *               only the partitions the window touches are read).
 *   dtype       ZR_BF16 (the 16-bit params) or ZR_FP32 (e.g. masters).
 * A pure copy: bit-exact. */
zr_status zr_all_gather_params(const zr_plan* plan, int32_t group,
                               const void* const* parts, zr_dtype dtype,
                               void* out, int64_t out_base, int64_t out_len,
                               hipStream_t stream);

/* zr_ring_ag_step -- one step of the ring all-gather phase with every card's
 * buffer resident here ([Megatron DP] "深入：all-reduce 底层算法（NCCL）", second
 * phase).  For every rank k: buf_k[c] = buf_{k-1}[c], c = (k - step - 1) mod
 * n_ranks.  After the n-1 reduce-scatter steps, steps 0..n_ranks-2 of this
 * phase leave every rank holding every reduced chunk (ring all-reduce). */
zr_status zr_ring_ag_step(float* const* rank_bufs, int32_t n_ranks,
                          int64_t chunk_numel, int32_t step,
                          hipStream_t stream);

/* ------------------------------------------------------------- errors --- */

/* Message for the last failed call on this thread ("" if none). */
const char* zr_last_error(void);
int zr_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ZR_H */
