// Host planner for partition-aware gradient reduction (plain C++17, no HIP).
//
// Builds, per reduction group, the flat parameter space padded to equal
// partitions, each param's partition ids and grad start offsets, and the
// buckets of at most reduce_bucket_size elements cut into merged
// (dst, bucket_offset, numel) slices.
//   [ZeRO-RS blog] §二: optimizer state / 16-bit grads split into
//     data-parallel-degree equal parts;
//   §三.2: per-param partition metadata (param_to_partition_ids,
//     grad_start_offset), slices keyed by destination, contiguous pieces with
//     one destination merged before the reduction;
//   §四: the IPG bucket is filled in gradient-ready (list) order;
//   §五: reduce_bucket_size caps the elements of one reduction.
//   §六: divisor dp_world_size / sequence_parallel_size; expert params use
//     their own (expert-data-parallel) group.
// A bucket boundary splits a param (the cap is a hard limit).  Padding sits at
// the end of each group's flat space and belongs to no bucket.

#include <algorithm>
#include <limits>
#include <new>

#include "zr_internal.h"

namespace zr {

namespace {
thread_local std::string g_last_error;

bool add_overflows(int64_t a, int64_t b) {
  return b > 0 && a > std::numeric_limits<int64_t>::max() - b;
}
bool mul_overflows(int64_t a, int64_t b) {
  return a > 0 && b > 0 && a > std::numeric_limits<int64_t>::max() / b;
}
}  // namespace

zr_status fail(zr_status st, const std::string& msg) {
  g_last_error = msg;
  return st;
}
void clear_error() { g_last_error.clear(); }

}  // namespace zr

using zr::fail;

extern "C" const char* zr_last_error(void) { return zr::g_last_error.c_str(); }
extern "C" int zr_version(void) { return ZR_VERSION; }

namespace {

zr_status build_plan(const zr_param* params, int64_t n_params,
                     const zr_group* groups, int32_t n_groups, int64_t B,
                     int32_t partition_gradients, int64_t align,
                     zr_plan* plan) {
  plan->bucket_size = B;
  plan->partition_gradients = partition_gradients;
  plan->groups.resize(n_groups);
  for (int32_t g = 0; g < n_groups; ++g) {
    const zr_group& in = groups[g];
    if (in.world <= 0 || in.sp <= 0)
      return fail(ZR_ERR_INVALID, "group " + std::to_string(g) +
                                      ": world and sp must be positive");
    if (in.world % in.sp != 0)
      return fail(ZR_ERR_INVALID, "group " + std::to_string(g) +
                                      ": sp must divide world");
    if (in.world > ZR_MAX_WORLD)
      return fail(ZR_ERR_INVALID, "group " + std::to_string(g) +
                                      ": world exceeds ZR_MAX_WORLD");
    plan->groups[g].world = in.world;
    plan->groups[g].sp = in.sp;
    plan->groups[g].divisor = in.world / in.sp;
  }

  // Flat offsets: params of one group are laid out contiguously in list order.
  plan->params.resize(n_params);
  int64_t list_total = 0;
  for (int64_t p = 0; p < n_params; ++p) {
    const zr_param& in = params[p];
    if (in.numel <= 0)
      return fail(ZR_ERR_INVALID, "param " + std::to_string(p) +
                                      ": numel must be positive");
    if (in.group < 0 || in.group >= n_groups)
      return fail(ZR_ERR_INVALID, "param " + std::to_string(p) +
                                      ": group index out of range");
    zr::GroupInfo& gi = plan->groups[in.group];
    if (zr::add_overflows(gi.total, in.numel) ||
        zr::add_overflows(list_total, in.numel))
      return fail(ZR_ERR_INVALID, "flat size overflows int64");
    plan->params[p].numel = in.numel;
    plan->params[p].group = in.group;
    plan->params[p].offset = gi.total;
    plan->params[p].list_pos = list_total;
    gi.total += in.numel;
    list_total += in.numel;
  }

  // Equal partitions: pad each group at its end to a multiple of world*align.
  for (int32_t g = 0; g < n_groups; ++g) {
    zr::GroupInfo& gi = plan->groups[g];
    if (zr::mul_overflows(gi.world, align))
      return fail(ZR_ERR_INVALID, "world*align overflows int64");
    const int64_t unit = gi.world * align;
    const int64_t units = gi.total / unit + (gi.total % unit != 0);
    if (zr::mul_overflows(units, unit))
      return fail(ZR_ERR_INVALID, "padded size overflows int64");
    gi.padded = units * unit;
    gi.part = gi.padded / gi.world;
  }

  // Partition ids and the start offset of each partition's piece in a param.
  for (auto& pi : plan->params) {
    const int64_t P = plan->groups[pi.group].part;
    const int64_t first = pi.offset / P;
    const int64_t last = (pi.offset + pi.numel - 1) / P;
    for (int64_t k = first; k <= last; ++k) {
      pi.partitions.push_back(static_cast<int32_t>(k));
      pi.start_offsets.push_back(std::max<int64_t>(0, k * P - pi.offset));
    }
  }

  // Buckets over the list, then pieces cut at bucket and partition borders;
  // consecutive pieces of one bucket with equal (group, dst) are merged.
  plan->num_buckets = list_total / B + (list_total % B != 0);
  plan->bucket_first.assign(plan->num_buckets + 1, 0);
  int64_t pos = 0;  // position in the list-ordered bucket space
  for (const auto& pi : plan->params) {
    const int64_t P = plan->groups[pi.group].part;
    int64_t f = pi.offset;
    const int64_t end = pi.offset + pi.numel;
    while (f < end) {
      const int64_t b = pos / B;
      const int32_t dst = static_cast<int32_t>(f / P);
      // Room left in this bucket and in this partition (no (b+1)*B products:
      // those could overflow for a huge B).
      const int64_t room = std::min({end - f, B - pos % B, P - f % P});
      zr_slice* last = plan->slices.empty() ? nullptr : &plan->slices.back();
      if (last && last->bucket == b && last->group == pi.group &&
          last->dst == dst) {
        last->numel += room;  // contiguous in both bucket and flat space
      } else {
        zr_slice s;
        s.bucket = b;
        s.group = pi.group;
        s.dst = dst;
        s.bucket_offset = pos - b * B;
        s.flat_offset = f;
        s.part_offset = f - static_cast<int64_t>(dst) * P;
        s.numel = room;
        plan->slices.push_back(s);
      }
      pos += room;
      f += room;
    }
  }
  // Index of the first slice of every bucket (slices are in bucket order).
  size_t i = 0;
  for (int64_t b = 0; b <= plan->num_buckets; ++b) {
    while (i < plan->slices.size() && plan->slices[i].bucket < b) ++i;
    plan->bucket_first[b] = static_cast<int64_t>(i);
  }
  return ZR_OK;
}

}  // namespace

extern "C" zr_status zr_plan_buckets(const zr_param* params, int64_t n_params,
                                     const zr_group* groups, int32_t n_groups,
                                     int64_t reduce_bucket_size,
                                     int32_t partition_gradients,
                                     int64_t align, zr_plan** out) {
  zr::clear_error();
  if (!out) return fail(ZR_ERR_INVALID, "out is null");
  if (n_params <= 0 || !params)
    return fail(ZR_ERR_INVALID, "need at least one param");
  if (n_groups <= 0 || !groups)
    return fail(ZR_ERR_INVALID, "need at least one group");
  if (reduce_bucket_size <= 0)
    return fail(ZR_ERR_INVALID, "reduce_bucket_size must be positive");
  if (align <= 0) return fail(ZR_ERR_INVALID, "align must be positive");
  if (partition_gradients != 0 && partition_gradients != 1)
    return fail(ZR_ERR_INVALID, "partition_gradients must be 0 or 1");
  zr_plan* plan = new (std::nothrow) zr_plan();
  if (!plan) return fail(ZR_ERR_OOM, "out of host memory");
  zr_status st;
  try {
    st = build_plan(params, n_params, groups, n_groups, reduce_bucket_size,
                    partition_gradients, align, plan);
  } catch (const std::bad_alloc&) {
    st = fail(ZR_ERR_OOM, "out of host memory");
  } catch (...) {
    st = fail(ZR_ERR_INVALID, "unexpected error while planning");
  }
  if (st != ZR_OK) {
    delete plan;
    return st;
  }
  *out = plan;
  return ZR_OK;
}

extern "C" void zr_plan_free(zr_plan* plan) {
  if (!plan) return;
  if (plan->dev && plan->dev_release) plan->dev_release(plan->dev);
  delete plan;
}

extern "C" zr_status zr_plan_num_buckets(const zr_plan* plan, int64_t* out) {
  if (!plan || !out) return fail(ZR_ERR_INVALID, "null argument");
  *out = plan->num_buckets;
  return ZR_OK;
}

extern "C" zr_status zr_plan_num_params(const zr_plan* plan, int64_t* out) {
  if (!plan || !out) return fail(ZR_ERR_INVALID, "null argument");
  *out = static_cast<int64_t>(plan->params.size());
  return ZR_OK;
}

extern "C" zr_status zr_plan_partition_gradients(const zr_plan* plan,
                                                 int32_t* out) {
  if (!plan || !out) return fail(ZR_ERR_INVALID, "null argument");
  *out = plan->partition_gradients;
  return ZR_OK;
}

extern "C" zr_status zr_plan_group_info(const zr_plan* plan, int32_t g,
                                        int64_t* total, int64_t* padded,
                                        int64_t* part_numel, float* divisor) {
  if (!plan) return fail(ZR_ERR_INVALID, "null plan");
  if (g < 0 || g >= static_cast<int32_t>(plan->groups.size()))
    return fail(ZR_ERR_INVALID, "group index out of range");
  const zr::GroupInfo& gi = plan->groups[g];
  if (total) *total = gi.total;
  if (padded) *padded = gi.padded;
  if (part_numel) *part_numel = gi.part;
  if (divisor) *divisor = static_cast<float>(gi.divisor);
  return ZR_OK;
}

extern "C" zr_status zr_plan_param_offset(const zr_plan* plan, int64_t p,
                                          int64_t* out) {
  if (!plan || !out) return fail(ZR_ERR_INVALID, "null argument");
  if (p < 0 || p >= static_cast<int64_t>(plan->params.size()))
    return fail(ZR_ERR_INVALID, "param index out of range");
  *out = plan->params[p].offset;
  return ZR_OK;
}

extern "C" zr_status zr_plan_param_partitions(const zr_plan* plan, int64_t p,
                                              const int32_t** ids,
                                              int32_t* n) {
  if (!plan || !ids || !n) return fail(ZR_ERR_INVALID, "null argument");
  if (p < 0 || p >= static_cast<int64_t>(plan->params.size()))
    return fail(ZR_ERR_INVALID, "param index out of range");
  *ids = plan->params[p].partitions.data();
  *n = static_cast<int32_t>(plan->params[p].partitions.size());
  return ZR_OK;
}

extern "C" zr_status zr_plan_grad_start_offset(const zr_plan* plan, int64_t p,
                                               int32_t k, int64_t* out) {
  if (!plan || !out) return fail(ZR_ERR_INVALID, "null argument");
  if (p < 0 || p >= static_cast<int64_t>(plan->params.size()))
    return fail(ZR_ERR_INVALID, "param index out of range");
  const auto& pi = plan->params[p];
  for (size_t i = 0; i < pi.partitions.size(); ++i)
    if (pi.partitions[i] == k) {
      *out = pi.start_offsets[i];
      return ZR_OK;
    }
  return fail(ZR_ERR_INVALID, "param does not touch that partition");
}

extern "C" zr_status zr_plan_param_buckets(const zr_plan* plan, int64_t p,
                                           int64_t* first, int64_t* last) {
  if (!plan || !first || !last) return fail(ZR_ERR_INVALID, "null argument");
  if (p < 0 || p >= static_cast<int64_t>(plan->params.size()))
    return fail(ZR_ERR_INVALID, "param index out of range");
  *first = plan->params[p].list_pos / plan->bucket_size;
  *last = (plan->params[p].list_pos + plan->params[p].numel - 1) / plan->bucket_size;
  return ZR_OK;
}

extern "C" zr_status zr_plan_slices(const zr_plan* plan, int64_t bucket,
                                    const zr_slice** s, int64_t* n) {
  if (!plan || !s || !n) return fail(ZR_ERR_INVALID, "null argument");
  if (bucket < -1 || bucket >= plan->num_buckets)
    return fail(ZR_ERR_INVALID, "bucket index out of range");
  if (bucket == -1) {
    *s = plan->slices.data();
    *n = static_cast<int64_t>(plan->slices.size());
  } else {
    const int64_t a = plan->bucket_first[bucket];
    *s = plan->slices.data() + a;
    *n = plan->bucket_first[bucket + 1] - a;
  }
  return ZR_OK;
}
