// combine.hip -- weighted gather-sum back to token order:
//   x_out[t,:] = sum_j expert_scales[t,j] * y[slot(t,j), :] + shared[t,:]
// (the formula of the npu_moe_distribute_combine page; the shared expert is
// added without a weight, as its expert_scales parameter note says).
//
// One workgroup per (token, row chunk).  The token's slots and scales are
// workgroup-uniform.  Each thread issues the K row loads of its 16-byte
// vector (plus the shared row) before consuming any, so K+1 independent
// 16-byte loads are in flight per thread; the sum is an fp32 fused
// multiply-add chain in ascending j from +0, then + shared, then one
// round-to-nearest-even into bf16.  y is read exactly once (non-temporal
// loads) and x_out written once (non-temporal stores).
#include "moe_internal.h"

namespace moe {
namespace {

template <int THREADS, int VPT, int KMAX>
__global__ __launch_bounds__(THREADS) void combine_kernel(
    const u32x4* __restrict__ y, int64_t ys, int64_t cap, const int32_t* __restrict__ ids,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ send,
    const float* __restrict__ scales, const u32x4* __restrict__ shared, int64_t ss,
    int32_t nvec, int32_t nchunks, int32_t k, int32_t E, u32x4* __restrict__ out,
    int32_t* status) {
  const int32_t t = blockIdx.x / nchunks;
  const int32_t chunk = blockIdx.x - t * nchunks;
  const int32_t v0 = chunk * (THREADS * VPT) + threadIdx.x;

  int64_t slot[KMAX];
  float w[KMAX];
  load_token_routes<KMAX>(t, ids, idx, send, scales, k, E, cap, slot, w, status,
                          threadIdx.x < kWave && chunk == 0);

#pragma unroll
  for (int jv = 0; jv < VPT; ++jv) {
    const int32_t v = v0 + jv * THREADS;
    if (v >= nvec) break;
    u32x4 yv[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (slot[j] >= 0) yv[j] = __builtin_nontemporal_load(y + slot[j] * ys + v);
    u32x4 sv = {0u, 0u, 0u, 0u};
    if (shared) sv = __builtin_nontemporal_load(shared + (int64_t)t * ss + v);

    float acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = 0.0f;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (slot[j] < 0) continue;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        acc[2 * c] = __builtin_fmaf(w[j], bf16lo_to_f32(yv[j][c]), acc[2 * c]);
        acc[2 * c + 1] = __builtin_fmaf(w[j], bf16hi_to_f32(yv[j][c]), acc[2 * c + 1]);
      }
    }
    if (shared) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        acc[2 * c] = acc[2 * c] + bf16lo_to_f32(sv[c]);
        acc[2 * c + 1] = acc[2 * c + 1] + bf16hi_to_f32(sv[c]);
      }
    }
    u32x4 o;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      o[c] = f32_to_bf16_rne(acc[2 * c]) | (f32_to_bf16_rne(acc[2 * c + 1]) << 16);
    __builtin_nontemporal_store(o, out + (int64_t)t * nvec + v);
  }
}

template <int THREADS, int VPT>
hipError_t launch_t(int kmax, dim3 grid, const u32x4* y, int64_t ys, int64_t cap,
                    const int32_t* ids, const int32_t* idx, const int32_t* send,
                    const float* scales, const u32x4* shared, int64_t ss, int32_t nvec,
                    int32_t nchunks, int32_t k, int32_t E, u32x4* out, int32_t* status,
                    hipStream_t stream) {
  switch (kmax) {
    case 2:
      combine_kernel<THREADS, VPT, 2><<<grid, THREADS, 0, stream>>>(
          y, ys, cap, ids, idx, send, scales, shared, ss, nvec, nchunks, k, E, out, status);
      break;
    case 4:
      combine_kernel<THREADS, VPT, 4><<<grid, THREADS, 0, stream>>>(
          y, ys, cap, ids, idx, send, scales, shared, ss, nvec, nchunks, k, E, out, status);
      break;
    case 8:
      combine_kernel<THREADS, VPT, 8><<<grid, THREADS, 0, stream>>>(
          y, ys, cap, ids, idx, send, scales, shared, ss, nvec, nchunks, k, E, out, status);
      break;
    default:
      combine_kernel<THREADS, VPT, 16><<<grid, THREADS, 0, stream>>>(
          y, ys, cap, ids, idx, send, scales, shared, ss, nvec, nchunks, k, E, out, status);
      break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(const void* y, int64_t y_stride, int64_t capacity_rows,
                          const int32_t* ids, const int32_t* expand_idx, const int32_t* send,
                          const float* scales, const void* shared, int64_t shared_stride,
                          int32_t bs, int32_t hidden, int32_t k, int32_t num_experts,
                          void* out, int32_t* status, hipStream_t stream) {
  constexpr int kThreads = 128;
  constexpr int kVpt = 1;
  const int32_t nvec = hidden / 8;
  const int32_t nchunks = (nvec + kThreads * kVpt - 1) / (kThreads * kVpt);
  const dim3 grid((uint32_t)((int64_t)bs * nchunks));
  const int kmax = k <= 2 ? 2 : k <= 4 ? 4 : k <= 8 ? 8 : 16;
  return launch_t<kThreads, kVpt>(kmax, grid, static_cast<const u32x4*>(y), y_stride / 8,
                                  capacity_rows, ids, expand_idx, send, scales,
                                  static_cast<const u32x4*>(shared), shared_stride / 8, nvec,
                                  nchunks, k, num_experts, static_cast<u32x4*>(out), status,
                                  stream);
}

}  // namespace moe
