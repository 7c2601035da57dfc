// dispatch.hip -- scatter token rows into the expert-contiguous buffer
// (bf16 bit copy, or e4m3 quantisation with one fp32 scale per 128 channels
// fused into the scatter).  The combine on the npu_moe_distribute_combine page
// retraces exactly this path; row slot(t,j) = ep_send_counts[e] + expand_idx.
//
// Work split: one workgroup per (token, chunk of the row).  The token's slots
// are workgroup-uniform (fetched lane-parallel, then broadcast to scalar
// registers), the row chunk is read once with
// 16-byte loads and written K times with 16-byte non-temporal stores (the
// dispatched rows are write-once streams).  Every destination row is checked
// against capacity_rows before any store.
#include "moe_internal.h"

namespace moe {
namespace {

template <int THREADS, int VPT, int KMAX>
__global__ __launch_bounds__(THREADS) void dispatch_bf16_kernel(
    const u32x4* __restrict__ x, int64_t xs, int32_t nvec, int32_t nchunks,
    const int32_t* __restrict__ ids, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ send, int32_t k, int32_t E, u32x4* __restrict__ out, int64_t os,
    int64_t cap, int32_t* status) {
  const int32_t t = blockIdx.x / nchunks;
  const int32_t chunk = blockIdx.x - t * nchunks;
  const int32_t v0 = chunk * (THREADS * VPT) + threadIdx.x;

  int64_t slot[KMAX];
  float unused_w[KMAX];
  load_token_routes<KMAX>(t, ids, idx, send, nullptr, k, E, cap, slot, unused_w, status,
                          threadIdx.x < kWave && chunk == 0);

  const u32x4* src = x + (int64_t)t * xs;
  u32x4 r[VPT];
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    const int32_t v = v0 + j * THREADS;
    if (v < nvec) r[j] = src[v];
  }
#pragma unroll
  for (int jj = 0; jj < KMAX; ++jj) {
    if (slot[jj] < 0) continue;
    u32x4* dst = out + slot[jj] * os;
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int32_t v = v0 + j * THREADS;
      if (v < nvec) __builtin_nontemporal_store(r[j], dst + v);
    }
  }
}

// Each thread owns 16 consecutive channels (two 16-byte loads of bf16, one
// 16-byte store of e4m3 codes); 8 neighbouring lanes form one 128-channel
// scale block and combine their maxima with cross-lane exchanges.
template <int THREADS, int KMAX>
__global__ __launch_bounds__(THREADS) void dispatch_fp8_kernel(
    const u32x4* __restrict__ x, int64_t xs, int32_t ngroups, int32_t nchunks,
    const int32_t* __restrict__ ids, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ send, int32_t k, int32_t E, u32x4* __restrict__ out, int64_t os,
    float* __restrict__ scales, int32_t nblk, int64_t cap, int32_t* status) {
  const int32_t t = blockIdx.x / nchunks;
  const int32_t chunk = blockIdx.x - t * nchunks;
  const int32_t g = chunk * THREADS + threadIdx.x;  // 16-channel group within the row
  const bool active = g < ngroups;

  int64_t slot[KMAX];
  float unused_w[KMAX];
  load_token_routes<KMAX>(t, ids, idx, send, nullptr, k, E, cap, slot, unused_w, status,
                          threadIdx.x < kWave && chunk == 0);

  u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
  if (active) {
    const u32x4* src = x + (int64_t)t * xs + 2 * (int64_t)g;
    a = src[0];
    b = src[1];
  }
  float f[16];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    f[2 * c] = bf16lo_to_f32(a[c]);
    f[2 * c + 1] = bf16hi_to_f32(a[c]);
    f[8 + 2 * c] = bf16lo_to_f32(b[c]);
    f[8 + 2 * c + 1] = bf16hi_to_f32(b[c]);
  }
  float amax = 0.0f;
#pragma unroll
  for (int c = 0; c < 16; ++c) amax = fmaxf(amax, fabsf(f[c]));
  amax = fmaxf(amax, __shfl_xor(amax, 1, kWave));
  amax = fmaxf(amax, __shfl_xor(amax, 2, kWave));
  amax = fmaxf(amax, __shfl_xor(amax, 4, kWave));

  const float s = amax / 448.0f;  // IEEE division (correctly rounded)
  u32x4 codes = {0u, 0u, 0u, 0u};
  if (amax != 0.0f) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float q0 = __builtin_amdgcn_fmed3f(f[4 * c + 0] / s, 448.0f, -448.0f);
      const float q1 = __builtin_amdgcn_fmed3f(f[4 * c + 1] / s, 448.0f, -448.0f);
      const float q2 = __builtin_amdgcn_fmed3f(f[4 * c + 2] / s, 448.0f, -448.0f);
      const float q3 = __builtin_amdgcn_fmed3f(f[4 * c + 3] / s, 448.0f, -448.0f);
      int w = __builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, 0, false);
      w = __builtin_amdgcn_cvt_pk_fp8_f32(q2, q3, w, true);
      codes[c] = (uint32_t)w;
    }
  }

  const bool writes_scale = active && (g & 7) == 0;
#pragma unroll
  for (int jj = 0; jj < KMAX; ++jj) {
    if (slot[jj] < 0) continue;
    if (active) __builtin_nontemporal_store(codes, out + slot[jj] * os + g);
    if (writes_scale) __builtin_nontemporal_store(s, scales + slot[jj] * nblk + (g >> 3));
  }
}

template <int THREADS, int VPT>
hipError_t launch_bf16_t(int kmax, dim3 grid, const u32x4* x, int64_t xs, int32_t nvec,
                         int32_t nchunks, const int32_t* ids, const int32_t* idx,
                         const int32_t* send, int32_t k, int32_t E, u32x4* out, int64_t os,
                         int64_t cap, int32_t* status, hipStream_t stream) {
  switch (kmax) {
    case 2:
      dispatch_bf16_kernel<THREADS, VPT, 2><<<grid, THREADS, 0, stream>>>(
          x, xs, nvec, nchunks, ids, idx, send, k, E, out, os, cap, status);
      break;
    case 4:
      dispatch_bf16_kernel<THREADS, VPT, 4><<<grid, THREADS, 0, stream>>>(
          x, xs, nvec, nchunks, ids, idx, send, k, E, out, os, cap, status);
      break;
    case 8:
      dispatch_bf16_kernel<THREADS, VPT, 8><<<grid, THREADS, 0, stream>>>(
          x, xs, nvec, nchunks, ids, idx, send, k, E, out, os, cap, status);
      break;
    default:
      dispatch_bf16_kernel<THREADS, VPT, 16><<<grid, THREADS, 0, stream>>>(
          x, xs, nvec, nchunks, ids, idx, send, k, E, out, os, cap, status);
      break;
  }
  return hipGetLastError();
}

template <int THREADS>
hipError_t launch_fp8_t(int kmax, dim3 grid, const u32x4* x, int64_t xs, int32_t ngroups,
                        int32_t nchunks, const int32_t* ids, const int32_t* idx,
                        const int32_t* send, int32_t k, int32_t E, u32x4* out, int64_t os,
                        float* scales, int32_t nblk, int64_t cap, int32_t* status,
                        hipStream_t stream) {
  switch (kmax) {
    case 2:
      dispatch_fp8_kernel<THREADS, 2><<<grid, THREADS, 0, stream>>>(
          x, xs, ngroups, nchunks, ids, idx, send, k, E, out, os, scales, nblk, cap, status);
      break;
    case 4:
      dispatch_fp8_kernel<THREADS, 4><<<grid, THREADS, 0, stream>>>(
          x, xs, ngroups, nchunks, ids, idx, send, k, E, out, os, scales, nblk, cap, status);
      break;
    case 8:
      dispatch_fp8_kernel<THREADS, 8><<<grid, THREADS, 0, stream>>>(
          x, xs, ngroups, nchunks, ids, idx, send, k, E, out, os, scales, nblk, cap, status);
      break;
    default:
      dispatch_fp8_kernel<THREADS, 16><<<grid, THREADS, 0, stream>>>(
          x, xs, ngroups, nchunks, ids, idx, send, k, E, out, os, scales, nblk, cap, status);
      break;
  }
  return hipGetLastError();
}

int kmax_for(int32_t k) { return k <= 2 ? 2 : k <= 4 ? 4 : k <= 8 ? 8 : 16; }

}  // namespace

hipError_t launch_dispatch_bf16(const void* x, int64_t x_stride, int32_t bs, int32_t hidden,
                                const int32_t* ids, const int32_t* expand_idx,
                                const int32_t* send, int32_t k, int32_t num_experts,
                                void* expand_x, int64_t expand_x_stride, int64_t capacity_rows,
                                int32_t* status, hipStream_t stream) {
  constexpr int kThreads = 128;
  constexpr int kVpt = 1;
  const int32_t nvec = hidden / 8;  // 16-byte vectors per row
  const int32_t nchunks = (nvec + kThreads * kVpt - 1) / (kThreads * kVpt);
  const dim3 grid((uint32_t)((int64_t)bs * nchunks));
  return launch_bf16_t<kThreads, kVpt>(kmax_for(k), grid, static_cast<const u32x4*>(x),
                                       x_stride / 8, nvec, nchunks, ids, expand_idx, send, k,
                                       num_experts, static_cast<u32x4*>(expand_x),
                                       expand_x_stride / 8, capacity_rows, status, stream);
}

hipError_t launch_dispatch_fp8(const void* x, int64_t x_stride, int32_t bs, int32_t hidden,
                               const int32_t* ids, const int32_t* expand_idx,
                               const int32_t* send, int32_t k, int32_t num_experts,
                               void* expand_x, int64_t expand_x_stride, int64_t capacity_rows,
                               float* quant_scales, int32_t* status, hipStream_t stream) {
  constexpr int kThreads = 64;
  const int32_t ngroups = hidden / 16;
  const int32_t nchunks = (ngroups + kThreads - 1) / kThreads;
  const dim3 grid((uint32_t)((int64_t)bs * nchunks));
  return launch_fp8_t<kThreads>(kmax_for(k), grid, static_cast<const u32x4*>(x), x_stride / 8,
                                ngroups, nchunks, ids, expand_idx, send, k, num_experts,
                                static_cast<u32x4*>(expand_x), expand_x_stride / 16,
                                quant_scales, hidden / 128, capacity_rows, status, stream);
}

}  // namespace moe
