/* Plain C client of libzr: builds the tiny workload's plan (params of 37,
 * 64*33 and 129 elements, one group of 4 replicas, reduce_bucket_size 1000)
 * through the C ABI only and prints it in the line format of
 * tests/golden/tiny_plan.txt.  Compiled as C (not C++) by the tests, so it
 * also checks that include/zr.h is a usable C header.  Host calls only. */
#include <stdio.h>

#include "zr.h"

static int check(zr_status st, const char* what) {
  if (st != ZR_OK) {
    fprintf(stderr, "%s failed (%d): %s\n", what, (int)st, zr_last_error());
    return 1;
  }
  return 0;
}

int main(void) {
  const zr_param params[3] = {{37, 0}, {64 * 33, 0}, {129, 0}};
  const zr_group group = {4, 1};
  zr_plan* plan = NULL;
  int64_t total = 0, padded = 0, part = 0, nb = 0, np = 0, ns = 0;
  float divisor = 0.0f;
  const zr_slice* sl = NULL;
  int64_t p, i;

  if (check(zr_plan_buckets(params, 3, &group, 1, 1000, 0, 1, &plan), "zr_plan_buckets"))
    return 1;
  if (check(zr_plan_group_info(plan, 0, &total, &padded, &part, &divisor), "group_info") ||
      check(zr_plan_num_buckets(plan, &nb), "num_buckets") ||
      check(zr_plan_num_params(plan, &np), "num_params"))
    return 1;
  printf("totals %lld %lld %lld %lld\n", (long long)total, (long long)padded,
         (long long)part, (long long)nb);
  for (p = 0; p < np; ++p) {
    int64_t off = 0, gso = 0;
    const int32_t* ids = NULL;
    int32_t n = 0, j;
    if (check(zr_plan_param_offset(plan, p, &off), "param_offset") ||
        check(zr_plan_param_partitions(plan, p, &ids, &n), "param_partitions"))
      return 1;
    printf("param %lld %lld ", (long long)p, (long long)off);
    for (j = 0; j < n; ++j) printf(j ? ";%d" : "%d", (int)ids[j]);
    printf(" ");
    for (j = 0; j < n; ++j) {
      if (check(zr_plan_grad_start_offset(plan, p, ids[j], &gso), "grad_start_offset"))
        return 1;
      printf(j ? ";%lld" : "%lld", (long long)gso);
    }
    printf("\n");
  }
  if (check(zr_plan_slices(plan, -1, &sl, &ns), "slices")) return 1;
  for (i = 0; i < ns; ++i)
    printf("slice %lld %d %lld %lld %lld %lld\n", (long long)sl[i].bucket, (int)sl[i].dst,
           (long long)sl[i].bucket_offset, (long long)sl[i].flat_offset,
           (long long)sl[i].part_offset, (long long)sl[i].numel);
  zr_plan_free(plan);
  return 0;
}
