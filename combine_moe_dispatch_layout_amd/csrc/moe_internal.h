// moe_internal.h -- declarations shared by the library's translation units:
// 16-byte vector type, bf16 helpers, and the kernel launchers that the C ABI
// in api.hip calls after validating its arguments.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe_dispatch.h"

namespace moe {

constexpr int kWave = 64;           // CDNA wavefront width
constexpr int kMaxExperts = 512;    // upper bound on num_experts
constexpr int kMaxTopK = 16;        // upper bound on k
constexpr int64_t kMaxRows = int64_t(1) << 30;  // bound on bs*k and on the padded total

// A 16-byte register vector; global loads/stores of this type become
// global_load_dwordx4 / global_store_dwordx4.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// bf16 held in the low / high half of a 32-bit word -> fp32 (exact).
__device__ __forceinline__ float bf16lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x0040u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Routes of token t: destination row slot[j] (-1 = pair skipped) and weight
// w[j] for j < KMAX.  Lanes 0..k-1 of every wave fetch one pair each (ids,
// expand_idx and scales in one round trip, send[e] in a second), then the
// values are broadcast to scalar registers, so the rest of the kernel
// branches on them uniformly.  A slot outside [0, cap) is reported through
// `status` when `report` is set (one lane group per token does it).
template <int KMAX>
__device__ __forceinline__ void load_token_routes(int32_t t, const int32_t* __restrict__ ids,
                                                  const int32_t* __restrict__ idx,
                                                  const int32_t* __restrict__ send,
                                                  const float* __restrict__ scales, int32_t k,
                                                  int32_t E, int64_t cap, int64_t (&slot)[KMAX],
                                                  float (&w)[KMAX], int32_t* status,
                                                  bool report) {
  const int lane = threadIdx.x & (kWave - 1);
  int64_t my_slot = -1;
  float my_w = 0.0f;
  if (lane < k) {
    const int64_t p = (int64_t)t * k + lane;
    const int e = ids[p];
    const int r = idx[p];
    if (scales) my_w = scales[p];
    if (e >= 0 && e < E && r >= 0) {
      const int64_t s = (int64_t)send[e] + r;
      if (s >= 0 && s < cap)
        my_slot = s;
      else if (report && status)
        atomicOr(status, (int)MOE_FLAG_GUARD);
    }
  }
  const int32_t lo = (int32_t)(my_slot & 0xFFFFFFFF);
  const int32_t hi = (int32_t)(my_slot >> 32);
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    const uint32_t l = (uint32_t)__builtin_amdgcn_readlane(lo, j);
    const int32_t h = __builtin_amdgcn_readlane(hi, j);
    slot[j] = (j < k) ? (int64_t)(((uint64_t)(uint32_t)h << 32) | l) : -1;
    w[j] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_w), j));
  }
}

// ---- layout ---------------------------------------------------------------
// Pairs ranked per workgroup and round trip parameters, chosen on the host.
struct LayoutPlan {
  int64_t n_pairs;          // bs * k
  int32_t blocks;           // workgroups of the ranking pass
  int32_t rounds;           // rounds of kLayoutThreads pairs per workgroup
  int64_t pairs_per_block;  // rounds * kLayoutThreads
};
constexpr int kLayoutWaves = 8;
constexpr int kLayoutThreads = kLayoutWaves * kWave;   // 512 pairs per round
constexpr int kLayoutSingleMaxRounds = 16;             // one workgroup up to 8192 pairs
constexpr int kLayoutMultiRounds = 8;                  // 4096 pairs per workgroup otherwise

LayoutPlan plan_layout(int32_t bs, int32_t k);
size_t layout_workspace_bytes(const LayoutPlan& p, int32_t num_experts);

hipError_t launch_layout(const int32_t* ids, int32_t k, int32_t num_experts, int32_t align,
                         const LayoutPlan& plan, int32_t* counts, int32_t* send,
                         int32_t* expand_idx, int32_t* status, void* workspace,
                         hipStream_t stream);

// ---- dispatch / combine -----------------------------------------------------
hipError_t launch_dispatch_bf16(const void* x, int64_t x_stride, int32_t bs, int32_t hidden,
                                const int32_t* ids, const int32_t* expand_idx,
                                const int32_t* send, int32_t k, int32_t num_experts,
                                void* expand_x, int64_t expand_x_stride, int64_t capacity_rows,
                                int32_t* status, hipStream_t stream);

hipError_t launch_dispatch_fp8(const void* x, int64_t x_stride, int32_t bs, int32_t hidden,
                               const int32_t* ids, const int32_t* expand_idx,
                               const int32_t* send, int32_t k, int32_t num_experts,
                               void* expand_x, int64_t expand_x_stride, int64_t capacity_rows,
                               float* quant_scales, int32_t* status, hipStream_t stream);

hipError_t launch_combine(const void* y, int64_t y_stride, int64_t capacity_rows,
                          const int32_t* ids, const int32_t* expand_idx, const int32_t* send,
                          const float* scales, const void* shared, int64_t shared_stride,
                          int32_t bs, int32_t hidden, int32_t k, int32_t num_experts,
                          void* out, int32_t* status, hipStream_t stream);

}  // namespace moe
