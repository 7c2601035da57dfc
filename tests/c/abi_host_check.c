/* Host-only check of the C ABI from plain C (C99): both headers compile as
 * C, the library links, and the calls that never reach the GPU behave as the
 * headers state (size queries, status strings, argument errors, the host
 * planner, binding and dropping timing events without launching).  Prints
 * "ok" and exits 0 on success. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "moe_dispatch.h"
#include "moe_probe.h"

static int failures = 0;

static void expect(int cond, const char* what) {
  if (!cond) {
    printf("FAILED: %s\n", what);
    ++failures;
  }
}

int main(void) {
  int32_t fake_ids = 0;
  int32_t counts[8], send[9], idx[8], moves[4 * 16], n_moves = -1;
  int64_t loads[2], before = 0, after = 0, ideal = 0;
  const int32_t expert_counts[4] = {1024, 0, 0, 0};

  expect(moe_abi_version() == 2, "abi version");
  expect(strcmp(moe_status_string(MOE_OK), "ok") == 0, "status string ok");
  expect(strstr(moe_status_string(99), "unknown") != NULL, "unknown status string");

  /* capacity: align * floor((n + (align-1)*min(E, n)) / align) */
  expect(moe_dispatch_capacity(16, 2, 8, 128) == 128 * ((32 + 127 * 8) / 128), "capacity tiny");
  expect(moe_dispatch_capacity(4096, 8, 256, 128) == 128 * ((32768 + 127 * 256) / 128),
         "capacity skewed");
  expect(moe_dispatch_capacity(4, 9, 8, 128) == -1, "capacity rejects k > E");
  expect(moe_dispatch_capacity(4, 2, 8, 3) == -1, "capacity rejects align not a power of 2");
  expect(moe_dispatch_layout_workspace_size(128, 8, 256) == 0, "one-workgroup workspace");
  expect(moe_dispatch_layout_workspace_size(16384, 8, 512) >= 64u * 512u * 4u,
         "multi-workgroup workspace");

  /* argument errors return before any launch */
  expect(moe_dispatch_layout(&fake_ids, 4, 0, 8, 128, counts, send, idx, NULL, NULL, 0, NULL) ==
             MOE_ERR_INVALID_ARG, "layout k = 0");
  expect(moe_dispatch_layout(&fake_ids, 16384, 8, 256, 128, counts, send, idx, NULL, NULL, 0,
                             NULL) == MOE_ERR_WORKSPACE, "layout without workspace");
  expect(moe_dispatch(NULL, 64, 4, 64, &fake_ids, idx, send, 2, 8, NULL, 64, 64, 7, NULL, NULL,
                      NULL) == MOE_ERR_UNSUPPORTED, "dispatch dtype");
  expect(moe_combine(NULL, 64, 64, &fake_ids, idx, send, NULL, NULL, 0, 4, 48, 2, 8, NULL, NULL,
                     NULL) == MOE_ERR_INVALID_ARG, "combine hidden % 32");
  expect(moe_combine(NULL, 64, 64, NULL, NULL, NULL, NULL, NULL, 0, 0, 64, 2, 8, NULL, NULL,
                     NULL) == MOE_OK, "combine of an empty batch");
  expect(moe_dispatch_fused(NULL, 64, 4, 64, &fake_ids, 2, 8, 128, counts, send, idx, NULL, 64,
                            64, 7, NULL, NULL, NULL, 0, NULL) == MOE_ERR_UNSUPPORTED,
         "fused dispatch dtype");
  expect(moe_dispatch_fused_replicated(NULL, 64, 4, 64, &fake_ids, 2, 8, NULL, NULL, 8, 0, 128,
                                       idx, counts, send, idx, NULL, 64, 64, MOE_BF16, NULL,
                                       NULL, NULL, 0, NULL) == MOE_ERR_INVALID_ARG,
         "replica-aware fused dispatch without its tables");

  /* measurement support: bindings are checked, and n = 0 drops them */
  {
    void* starts[2] = {(void*)&fake_ids, NULL};
    void* stops[2] = {(void*)&fake_ids, (void*)&fake_ids};
    expect(moe_time_next_launches(starts, stops, 17) == MOE_ERR_INVALID_ARG, "timing: n > 16");
    expect(moe_time_next_launches(starts, stops, 2) == MOE_ERR_INVALID_ARG,
           "timing: NULL event");
    expect(moe_time_unused_launches() == 0, "timing: nothing bound after errors");
    expect(moe_time_next_launches(starts, stops, 1) == MOE_OK, "timing: bind one pair");
    expect(moe_time_unused_launches() == 1, "timing: one pair bound");
    expect(moe_time_next_launches(NULL, NULL, 0) == MOE_OK, "timing: drop");
    expect(moe_time_unused_launches() == 0, "timing: dropped");
  }
  expect(moe_probe_stream_mix(NULL, 0, NULL, 0, 4, 24, 1, 8, NULL, NULL, NULL) ==
             MOE_ERR_INVALID_ARG, "probe row bytes not a multiple of 16");

  /* planner: one hot expert of 1024 rows between two ranks splits evenly */
  expect(moe_plan_compensation(expert_counts, 4, 2, 8, 10, 0, 16, moves, &n_moves, loads, &before,
                               &after, &ideal) == MOE_OK, "planner status");
  expect(n_moves == 1 && moves[0] == 0 && moves[1] == 0 && moves[2] == 1 && moves[3] == 512,
         "planner move");
  expect(loads[0] == 42 && loads[1] == 42 && before == 74 && after == 42, "planner loads");
  expect(moe_plan_compensation(expert_counts, 4, 3, 8, 10, 0, 16, moves, &n_moves, loads, NULL,
                               NULL, NULL) == MOE_ERR_INVALID_ARG, "planner uneven ranks");

  if (failures == 0) printf("ok\n");
  return failures == 0 ? 0 : 1;
}
