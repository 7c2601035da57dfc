/* The MoE path from plain C on the GPU, with no Python or torch: device
 * memory from the HIP runtime's C API, then moe_dispatch_layout ->
 * moe_dispatch -> moe_combine (and moe_dispatch_fused) through the C ABI.
 *
 * Check: with identity experts (the combine reads the dispatched rows back),
 * no shared row and weights that are exact binary fractions summing to 1,
 * every product and partial sum is exact in fp32, so the combine must return
 * x bit for bit.  Also: counts sum to bs*k, offsets are 128-aligned, status
 * is clear.  Cases cover the separate calls with one- and two-launch
 * layouts, moe_dispatch_fused (one launch, and layout launches with the rows
 * read ahead), moe_dispatch_fused_replicated over two replicas per expert,
 * and kernel times taken through moe_time_next_launches with HIP events of
 * the runtime's C API.  Prints "ok" and exits 0 on success.
 *
 * Build: gcc -std=c99 -D__HIP_PLATFORM_AMD__ -I include -I /opt/rocm/include
 *        abi_gpu_roundtrip.c libmoe_dispatch.so -L/opt/rocm/lib -lamdhip64 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "moe_dispatch.h"
#include "moe_probe.h"

static uint32_t lcg_state = 12345u;
static uint32_t lcg(void) {
  lcg_state = lcg_state * 1664525u + 1013904223u;
  return lcg_state >> 8;
}

/* bf16 bits of v, for values exactly representable in bf16 */
static uint16_t bf16_bits(float v) {
  uint32_t u;
  memcpy(&u, &v, 4);
  return (uint16_t)(u >> 16);
}

#define CHECK_HIP(call)                                                      \
  do {                                                                       \
    hipError_t e_ = (call);                                                  \
    if (e_ != hipSuccess) {                                                  \
      printf("HIP error %d at %s:%d\n", (int)e_, __FILE__, __LINE__);        \
      return 1;                                                              \
    }                                                                        \
  } while (0)

#define CHECK_MOE(call)                                                      \
  do {                                                                       \
    int s_ = (call);                                                         \
    if (s_ != MOE_OK) {                                                      \
      printf("moe status %d (%s) at line %d\n", s_, moe_status_string(s_),   \
             __LINE__);                                                      \
      return 1;                                                              \
    }                                                                        \
  } while (0)

/* path: 0 = separate calls, 1 = moe_dispatch_fused, 2 = moe_dispatch_fused_replicated
 * with two equally likely replicas per expert (dispatch and combine then run
 * over the 2e replicas), 3 = moe_dispatch_fused with every kernel timed by
 * events bound through moe_time_next_launches. */
static int run_case(int32_t bs, int32_t hidden, int32_t e, int32_t k, int path) {
  const int64_t n = (int64_t)bs * k;
  const int32_t ranked = path == 2 ? 2 * e : e;  /* experts the layout ranks over */
  const int64_t cap = moe_dispatch_capacity(bs, k, ranked, 128);
  const size_t ws_bytes = moe_dispatch_layout_workspace_size(bs, k, ranked);
  int32_t* ids = malloc(sizeof(int32_t) * n);
  float* scales = malloc(sizeof(float) * n);
  uint16_t* x = malloc(sizeof(uint16_t) * bs * hidden);
  uint16_t* out = malloc(sizeof(uint16_t) * bs * hidden);
  int32_t* counts = malloc(sizeof(int32_t) * ranked);
  int32_t* send = malloc(sizeof(int32_t) * (ranked + 1));
  int32_t* offsets = malloc(sizeof(int32_t) * (e + 1));
  uint32_t* thresholds = malloc(sizeof(uint32_t) * 2 * e);
  int32_t status = -1;
  if (!ids || !scales || !x || !out || !counts || !send || !offsets || !thresholds || cap <= 0)
    return 1;
  for (int32_t i = 0; i <= e; ++i) offsets[i] = 2 * i;
  for (int32_t i = 0; i < e; ++i) {
    thresholds[2 * i] = 0x7FFFFFFFu;
    thresholds[2 * i + 1] = 0xFFFFFFFFu;
  }

  /* distinct experts per row: k consecutive experts from a random start */
  for (int32_t t = 0; t < bs; ++t) {
    const int32_t start = (int32_t)(lcg() % (uint32_t)e);
    for (int32_t j = 0; j < k; ++j) ids[t * k + j] = (start + j) % e;
    /* weights 1/2, 1/4, ..., with the last one repeated so they sum to 1 */
    float w = 0.5f, sum = 0.0f;
    for (int32_t j = 0; j < k; ++j) {
      scales[t * k + j] = (j == k - 1) ? 1.0f - sum : w;
      sum += w;
      w *= 0.5f;
    }
  }
  for (int64_t i = 0; i < (int64_t)bs * hidden; ++i)
    x[i] = bf16_bits((float)((int32_t)(lcg() % 255u) - 127) / 64.0f);

  int32_t *d_ids, *d_counts, *d_send, *d_idx, *d_status, *d_rep, *d_off;
  uint32_t* d_thr;
  float* d_scales;
  void *d_x, *d_ex, *d_out, *d_ws = NULL;
  CHECK_HIP(hipMalloc((void**)&d_ids, sizeof(int32_t) * n));
  CHECK_HIP(hipMalloc((void**)&d_rep, sizeof(int32_t) * n));
  CHECK_HIP(hipMalloc((void**)&d_off, sizeof(int32_t) * (e + 1)));
  CHECK_HIP(hipMalloc((void**)&d_thr, sizeof(uint32_t) * 2 * e));
  CHECK_HIP(hipMalloc((void**)&d_scales, sizeof(float) * n));
  CHECK_HIP(hipMalloc((void**)&d_counts, sizeof(int32_t) * ranked));
  CHECK_HIP(hipMalloc((void**)&d_send, sizeof(int32_t) * (ranked + 1)));
  CHECK_HIP(hipMalloc((void**)&d_idx, sizeof(int32_t) * n));
  CHECK_HIP(hipMalloc((void**)&d_status, sizeof(int32_t)));
  CHECK_HIP(hipMalloc(&d_x, sizeof(uint16_t) * bs * hidden));
  CHECK_HIP(hipMalloc(&d_ex, sizeof(uint16_t) * cap * hidden));
  CHECK_HIP(hipMalloc(&d_out, sizeof(uint16_t) * bs * hidden));
  if (ws_bytes > 0) {
    CHECK_HIP(hipMalloc(&d_ws, ws_bytes));
    CHECK_HIP(hipMemset(d_ws, 0, ws_bytes)); /* zero-filled before its first use */
  }
  CHECK_HIP(hipMemcpy(d_ids, ids, sizeof(int32_t) * n, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(d_scales, scales, sizeof(float) * n, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(d_x, x, sizeof(uint16_t) * bs * hidden, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(d_off, offsets, sizeof(int32_t) * (e + 1), hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(d_thr, thresholds, sizeof(uint32_t) * 2 * e, hipMemcpyHostToDevice));

  hipEvent_t ev[8];
  void* ev_start[4];
  void* ev_stop[4];
  int timed = 0;
  const int32_t* route = d_ids;  /* the ids dispatch and combine take */
  if (path == 3) {
    for (int i = 0; i < 8; ++i) CHECK_HIP(hipEventCreate(&ev[i]));
    for (int i = 0; i < 4; ++i) {
      ev_start[i] = (void*)ev[2 * i];
      ev_stop[i] = (void*)ev[2 * i + 1];
    }
    CHECK_MOE(moe_time_next_launches(ev_start, ev_stop, 4));
  }
  if (path == 1 || path == 3) {
    CHECK_MOE(moe_dispatch_fused(d_x, hidden, bs, hidden, d_ids, k, e, 128, d_counts, d_send,
                                 d_idx, d_ex, hidden, cap, MOE_BF16, NULL, d_status, d_ws,
                                 ws_bytes, NULL));
  } else if (path == 2) {
    CHECK_MOE(moe_dispatch_fused_replicated(d_x, hidden, bs, hidden, d_ids, k, e, d_off, d_thr,
                                            2 * e, 77, 128, d_rep, d_counts, d_send, d_idx, d_ex,
                                            hidden, cap, MOE_BF16, NULL, d_status, d_ws, ws_bytes,
                                            NULL));
    route = d_rep;
  } else {
    CHECK_MOE(moe_dispatch_layout(d_ids, bs, k, e, 128, d_counts, d_send, d_idx, d_status, d_ws,
                                  ws_bytes, NULL));
    CHECK_MOE(moe_dispatch(d_x, hidden, bs, hidden, d_ids, d_idx, d_send, k, e, d_ex, hidden,
                           cap, MOE_BF16, NULL, d_status, NULL));
  }
  CHECK_MOE(moe_combine(d_ex, hidden, cap, route, d_idx, d_send, d_scales, NULL, 0, bs, hidden,
                        k, ranked, d_out, d_status, NULL));
  CHECK_HIP(hipDeviceSynchronize());
  if (path == 3) {
    /* the fused call launches one kernel at this size or two above 2048
       pairs (ranking with its scan, then the scatter), the combine one:
       every taken pair holds a positive kernel time */
    timed = 4 - moe_time_unused_launches();
    CHECK_MOE(moe_time_next_launches(NULL, NULL, 0));
    for (int i = 0; i < timed; ++i) {
      float ms = -1.0f;
      CHECK_HIP(hipEventElapsedTime(&ms, ev[2 * i], ev[2 * i + 1]));
      if (!(ms > 0.0f)) {
        printf("launch %d: kernel time %f ms\n", i, ms);
        return 1;
      }
    }
    for (int i = 0; i < 8; ++i) hipEventDestroy(ev[i]);
  }
  CHECK_HIP(hipMemcpy(out, d_out, sizeof(uint16_t) * bs * hidden, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(counts, d_counts, sizeof(int32_t) * ranked, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(send, d_send, sizeof(int32_t) * (ranked + 1), hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(&status, d_status, sizeof(int32_t), hipMemcpyDeviceToHost));

  int bad = 0;
  int64_t total = 0;
  for (int32_t i = 0; i < ranked; ++i) {
    total += counts[i];
    if (send[i] % 128 != 0 || send[i + 1] - send[i] < counts[i]) bad = 1;
  }
  if (total != n || status != 0) bad = 1;
  if (memcmp(out, x, sizeof(uint16_t) * bs * hidden) != 0) bad = 1;
  if (path == 3 && timed != (n <= 2048 ? 2 : 3)) bad = 1;
  static const char* names[] = {"separate", "fused", "fused replicated", "fused, timed"};
  printf("case bs=%d H=%d E=%d K=%d %s: %s\n", bs, hidden, e, k, names[path],
         bad ? "MISMATCH" : "round trip exact");

  hipFree(d_ids); hipFree(d_rep); hipFree(d_off); hipFree(d_thr);
  hipFree(d_scales); hipFree(d_counts); hipFree(d_send); hipFree(d_idx);
  hipFree(d_status); hipFree(d_x); hipFree(d_ex); hipFree(d_out);
  if (d_ws) hipFree(d_ws);
  free(ids); free(scales); free(x); free(out); free(counts); free(send); free(offsets);
  free(thresholds);
  return bad;
}

int main(void) {
  int bad = 0;
  bad |= run_case(37, 256, 16, 4, 0);    /* one layout workgroup */
  bad |= run_case(700, 512, 64, 8, 0);   /* workspace, two layout launches */
  bad |= run_case(128, 1024, 256, 8, 1); /* fused, one launch */
  bad |= run_case(600, 512, 64, 8, 1);   /* fused, ranking launch with read-ahead */
  bad |= run_case(300, 256, 32, 4, 2);   /* replica-aware fused, 64 replicas, one layout launch */
  bad |= run_case(900, 512, 128, 8, 2);  /* replica-aware fused, 256 replicas, read-ahead */
  bad |= run_case(128, 1024, 256, 8, 3); /* timed: one fused launch + combine */
  bad |= run_case(600, 512, 64, 8, 3);   /* timed: ranking + scan, scatter + combine */
  if (!bad) printf("ok\n");
  return bad;
}
