/* Plain C client of libzr: invalid calls return the documented status with a
 * message from zr_last_error(), before anything is enqueued (host-side
 * validation only; no device memory is touched and no GPU is needed).
 * Prints one line per check and exits non-zero on the first failure. */
#include <stdio.h>
#include <string.h>

#include "zr.h"

static int fails = 0;

static void expect(const char* what, zr_status got, zr_status want, const char* needle) {
  const char* msg = zr_last_error();
  int ok = got == want && (needle == NULL || (msg && strstr(msg, needle)));
  printf("%s %s: status %d, message \"%s\"\n", ok ? "ok" : "FAIL", what, (int)got,
         msg ? msg : "(null)");
  if (!ok) ++fails;
}

int main(void) {
  const zr_param params[3] = {{37, 0}, {64 * 33, 0}, {129, 0}};
  const zr_group group = {4, 1};
  const zr_group too_wide = {ZR_MAX_WORLD + 1, 1};
  const zr_group bad_sp = {4, 3};
  zr_plan* plan = NULL;
  zr_plan* none = NULL;

  expect("world above ZR_MAX_WORLD",
         zr_plan_buckets(params, 3, &too_wide, 1, 1000, 0, 1, &none), ZR_ERR_INVALID, NULL);
  expect("sp not dividing world",
         zr_plan_buckets(params, 3, &bad_sp, 1, 1000, 0, 1, &none), ZR_ERR_INVALID, NULL);
  expect("bucket size 0", zr_plan_buckets(params, 3, &group, 1, 0, 0, 1, &none),
         ZR_ERR_INVALID, NULL);
  expect("null output", zr_plan_buckets(params, 3, &group, 1, 1000, 0, 1, NULL),
         ZR_ERR_INVALID, NULL);
  if (none != NULL) {
    printf("FAIL a rejected plan was returned\n");
    ++fails;
  }
  expect("valid plan", zr_plan_buckets(params, 3, &group, 1, 1000, 0, 1, &plan), ZR_OK, NULL);
  if (!plan) return 1;

  int64_t v = 0;
  expect("param index out of range", zr_plan_param_offset(plan, 3, &v), ZR_ERR_INVALID, NULL);
  expect("partition the param does not touch",
         zr_plan_grad_start_offset(plan, 0, 2, &v), ZR_ERR_INVALID, NULL);

  /* Kernel entry points: validation fails before any HIP call. */
  const zr_replica reps[4] = {{(const void*)0x1000, 0, 2280}, {(const void*)0x2000, 0, 2280},
                              {(const void*)0x3000, 0, 2280}, {(const void*)0x4000, 0, 2280}};
  float* outs[4] = {(float*)0x100000, (float*)0x200000, (float*)0x300000, (float*)0x400000};
  expect("reduce: group out of range",
         zr_reduce_scatter_local(plan, 1, -1, -1, reps, ZR_FP32, outs, NULL), ZR_ERR_INVALID,
         "group");
  expect("reduce: bucket out of range",
         zr_reduce_scatter_local(plan, 0, 3, -1, reps, ZR_FP32, outs, NULL), ZR_ERR_INVALID,
         "bucket");
  expect("reduce: null replicas",
         zr_reduce_scatter_local(plan, 0, -1, -1, NULL, ZR_FP32, outs, NULL), ZR_ERR_INVALID,
         NULL);
  expect("reduce: unknown dtype",
         zr_reduce_scatter_local(plan, 0, -1, -1, reps, (zr_dtype)7, outs, NULL),
         ZR_ERR_INVALID, NULL);
  zr_adam h = {1e-3, 0.9, 0.999, 1e-8, 1};
  expect("fused: dst past the last partition",
         zr_reduce_scatter_adam(plan, 0, -1, 4, reps, ZR_FP32, &h, outs[0], outs[1], outs[2],
                                NULL, NULL, NULL),
         ZR_ERR_INVALID, "dst");
  h.step = 0;
  expect("fused: step 0",
         zr_reduce_scatter_adam(plan, 0, -1, 0, reps, ZR_FP32, &h, outs[0], outs[1], outs[2],
                                NULL, NULL, NULL),
         ZR_ERR_INVALID, "step");
  h.step = 1;
  expect("capped fused: no workgroups",
         zr_reduce_scatter_adam_capped(plan, 0, -1, 0, reps, ZR_FP32, &h, outs[0], outs[1],
                                       outs[2], NULL, NULL, 0, NULL),
         ZR_ERR_INVALID, "max_workgroups");
  expect("capped fused: dst past the last partition",
         zr_reduce_scatter_adam_capped(plan, 0, -1, 4, reps, ZR_FP32, &h, outs[0], outs[1],
                                       outs[2], NULL, NULL, 64, NULL),
         ZR_ERR_INVALID, "dst");
  expect("adam: negative n",
         zr_adam_partition(&h, outs[0], outs[1], outs[2], outs[3], NULL, -1, NULL),
         ZR_ERR_INVALID, "n must");
  float* rank_bufs[2] = {(float*)0x100000, (float*)0x100000};
  expect("ring: overlapping rank buffers", zr_ring_rs_step(rank_bufs, 2, 16, 0, NULL),
         ZR_ERR_INVALID, "overlap");
  expect("ring: one rank", zr_ring_rs_step(rank_bufs, 1, 16, 0, NULL), ZR_ERR_INVALID, NULL);

  zr_plan_free(plan);
  printf("%s\n", fails ? "FAILED" : "all ok");
  return fails ? 1 : 0;
}
