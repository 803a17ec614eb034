// Internal declarations shared by the host planner (zr_plan.cpp, plain C++)
// and the HIP translation unit (zr_kernels.hip).  Not part of the ABI.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "zr.h"

namespace zr {

// Sets the thread-local message returned by zr_last_error and returns `st`.
zr_status fail(zr_status st, const std::string& msg);
void clear_error();

struct GroupInfo {
  int32_t world = 0;     // R_g
  int32_t sp = 0;        // sp_g
  int64_t total = 0;     // T_g
  int64_t padded = 0;    // L_g
  int64_t part = 0;      // P_g
  int32_t divisor = 0;   // D_g = R_g / sp_g
};

struct ParamInfo {
  int64_t numel = 0;
  int32_t group = 0;
  int64_t offset = 0;                 // o_p in the group's flat space
  int64_t list_pos = 0;               // position in the list-ordered bucket space
  std::vector<int32_t> partitions;    // param_to_partition_ids
  std::vector<int64_t> start_offsets; // grad_start_offset, aligned with above
};

}  // namespace zr

// The plan object behind the opaque zr_plan handle.
struct zr_plan {
  std::vector<zr::GroupInfo> groups;
  std::vector<zr::ParamInfo> params;
  std::vector<zr_slice> slices;          // bucket order
  std::vector<int64_t> bucket_first;     // slices of bucket b: [first[b], first[b+1])
  int64_t bucket_size = 0;
  int64_t num_buckets = 0;
  int32_t partition_gradients = 0;

  // Device-side state owned by the HIP translation unit (lazily built launch
  // tables); released through dev_release when the plan is freed.
  void* dev = nullptr;
  void (*dev_release)(void*) = nullptr;
};
