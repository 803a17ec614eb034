// Randomised exercise of the host planner and its queries, built with
// AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_planner_sanitizers.py.
// Checks the plan's own invariants (slices tile every bucket, every element of
// every group lies in exactly one slice) and that invalid inputs are rejected.
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "zr.h"

#define REQUIRE(c)                                                    \
  do {                                                                \
    if (!(c)) {                                                       \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      return 1;                                                       \
    }                                                                 \
  } while (0)

int main(int argc, char** argv) {
  const int iters = argc > 1 ? std::atoi(argv[1]) : 300;
  std::mt19937_64 rng(12345);
  auto uni = [&](int64_t lo, int64_t hi) {
    return std::uniform_int_distribution<int64_t>(lo, hi)(rng);
  };
  for (int it = 0; it < iters; ++it) {
    const int ng = static_cast<int>(uni(1, 3));
    std::vector<zr_group> groups(ng);
    for (auto& g : groups) {
      g.sp = static_cast<int32_t>(uni(1, 3));
      g.world = g.sp * static_cast<int32_t>(uni(1, 8));
    }
    const int np = static_cast<int>(uni(1, 40));
    std::vector<zr_param> params(np);
    for (auto& p : params) {
      p.numel = uni(1, uni(0, 1) ? 50 : 5000);
      p.group = static_cast<int32_t>(uni(0, ng - 1));
    }
    const int64_t B = uni(1, 3) == 1 ? 1 : uni(1, 10000);
    const int64_t align = uni(1, 3) == 1 ? uni(1, 64) : 1;
    zr_plan* plan = nullptr;
    REQUIRE(zr_plan_buckets(params.data(), np, groups.data(), ng, B, 0, align, &plan) == ZR_OK);
    int64_t nb = 0, n = 0;
    REQUIRE(zr_plan_num_buckets(plan, &nb) == ZR_OK);
    const zr_slice* all = nullptr;
    REQUIRE(zr_plan_slices(plan, -1, &all, &n) == ZR_OK);
    // buckets are tiled in order by their slices
    int64_t seen = 0;
    for (int64_t b = 0; b < nb; ++b) {
      const zr_slice* s = nullptr;
      int64_t k = 0;
      REQUIRE(zr_plan_slices(plan, b, &s, &k) == ZR_OK);
      int64_t pos = 0;
      for (int64_t i = 0; i < k; ++i) {
        REQUIRE(s[i].bucket == b && s[i].bucket_offset == pos && s[i].numel > 0);
        pos += s[i].numel;
      }
      REQUIRE(b == nb - 1 || pos == B);
      seen += k;
    }
    REQUIRE(seen == n);
    // every element of every group in exactly one slice
    for (int g = 0; g < ng; ++g) {
      int64_t total = 0, padded = 0, part = 0;
      float div = 0;
      REQUIRE(zr_plan_group_info(plan, g, &total, &padded, &part, &div) == ZR_OK);
      REQUIRE(padded % groups[g].world == 0 && part * groups[g].world == padded);
      std::vector<unsigned char> cover(static_cast<size_t>(total), 0);
      for (int64_t i = 0; i < n; ++i) {
        if (all[i].group != g) continue;
        REQUIRE(all[i].flat_offset == int64_t(all[i].dst) * part + all[i].part_offset);
        REQUIRE(all[i].part_offset + all[i].numel <= part);
        for (int64_t f = all[i].flat_offset; f < all[i].flat_offset + all[i].numel; ++f) {
          REQUIRE(f < total && cover[f] == 0);
          cover[f] = 1;
        }
      }
      for (auto c : cover) REQUIRE(c == 1);
    }
    for (int p = 0; p < np; ++p) {
      int64_t off = 0, first = 0, last = 0;
      REQUIRE(zr_plan_param_offset(plan, p, &off) == ZR_OK);
      REQUIRE(zr_plan_param_buckets(plan, p, &first, &last) == ZR_OK && first <= last);
      const int32_t* ids = nullptr;
      int32_t k = 0;
      REQUIRE(zr_plan_param_partitions(plan, p, &ids, &k) == ZR_OK && k >= 1);
      for (int32_t i = 0; i < k; ++i) {
        int64_t gso = -1;
        REQUIRE(zr_plan_grad_start_offset(plan, p, ids[i], &gso) == ZR_OK);
        REQUIRE(gso >= 0 && gso < params[p].numel);
      }
      int64_t dummy = 0;
      REQUIRE(zr_plan_grad_start_offset(plan, p, ids[k - 1] + 1, &dummy) == ZR_ERR_INVALID);
    }
    int64_t dummy = 0;
    REQUIRE(zr_plan_param_offset(plan, np, &dummy) == ZR_ERR_INVALID);
    REQUIRE(zr_plan_slices(plan, nb, &all, &n) == ZR_ERR_INVALID);
    zr_plan_free(plan);
  }
  // invalid inputs are rejected and leave *out untouched
  zr_param bad{0, 0};
  zr_group g2{2, 1};
  zr_plan* untouched = reinterpret_cast<zr_plan*>(0x1);
  REQUIRE(zr_plan_buckets(&bad, 1, &g2, 1, 10, 0, 1, &untouched) == ZR_ERR_INVALID);
  REQUIRE(untouched == reinterpret_cast<zr_plan*>(0x1));
  zr_param huge[2] = {{int64_t(1) << 62, 0}, {int64_t(1) << 62, 0}};
  REQUIRE(zr_plan_buckets(huge, 2, &g2, 1, 10, 0, 1, &untouched) == ZR_ERR_INVALID);
  zr_plan_free(nullptr);
  std::printf("planner fuzz ok: %d random plans\n", iters);
  return 0;
}
