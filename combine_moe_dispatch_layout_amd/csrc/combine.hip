// combine.hip -- weighted gather-sum back to token order:
//   x_out[t,:] = sum_j expert_scales[t,j] * y[slot(t,j), :] + shared[t,:]
// (the formula of the npu_moe_distribute_combine page; the shared expert is
// added without a weight, as its expert_scales parameter note says).
//
// One workgroup per item = (token, row chunk).  The workgroup stages the
// send counts in LDS while lanes 0..K-1 fetch the token's ids / ranks /
// weights, so the routes cost one memory round trip plus one LDS read; the
// shared row's loads do not depend on them and go out with them.  Each
// thread then issues the K row loads of its 16-byte vector before consuming
// any, so K+1 independent 16-byte loads are in flight per thread.  The sum
// is an fp32 fused multiply-add chain in ascending j from +0, then + shared,
// then one round-to-nearest-even into bf16.  y is read exactly once
// (non-temporal loads) and x_out written once (non-temporal stores).
#include "moe_internal.h"

namespace moe {
namespace {

// The send counts' loads and the shared row's go out together and staging
// is one round trip (the decode step in graphs went from 14.6 to 12.9 us;
// staging one load at a time, as the scatter does in large grids, changed
// the 4096- and 16384-token combines by less than their run-to-run spread).
template <int THREADS, int VPT, int KMAX>
__global__ __launch_bounds__(THREADS) void combine_kernel(
    const u32x4* __restrict__ y, int64_t ys, int64_t cap, const int32_t* __restrict__ ids,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ send,
    const float* __restrict__ scales, const u32x4* shared, int64_t ss,
    int32_t nvec, int32_t nchunks, int32_t k, int32_t E,
    u32x4* __restrict__ out, int32_t* status) {
  __shared__ int send_lds[StagedSend<THREADS>::kSlots];
  const int32_t t = blockIdx.x / nchunks;
  const int32_t chunk = blockIdx.x - t * nchunks;
  PairMeta meta;
  fetch_pair_meta(meta, t, k, ids, idx, scales);
  // The shared row does not depend on the routes.  Every lane loads it (a
  // lane past the row end repeats its last vector, and without a shared row
  // all lanes read a zero vector), so no branch separates these loads from
  // the send counts' loads.
  const int32_t v0 = chunk * (THREADS * VPT) + threadIdx.x;
  u32x4 sv[VPT];
  StagedSend<THREADS> staged;
  staged.load(send, E + 1);
#pragma unroll
  for (int jv = 0; jv < VPT; ++jv) {
    const int32_t v = min(v0 + jv * THREADS, nvec - 1);
    sv[jv] = load_stream(shared ? shared + (int64_t)t * ss + v : &kZeroVec);
  }
  keep_order();
  staged.store(send_lds);
  __syncthreads();
  int64_t slot[KMAX];
  float w[KMAX];
  resolve_routes<KMAX>(meta, send_lds, nullptr, k, E, cap, slot, w, status,
                       threadIdx.x < kWave && chunk == 0);

  u32x4 yv[VPT][KMAX];
#pragma unroll
  for (int jv = 0; jv < VPT; ++jv) {
    const int32_t v = v0 + jv * THREADS;
    if (v < nvec) {
#pragma unroll
      for (int j = 0; j < KMAX; ++j)
        if (slot[j] >= 0) yv[jv][j] = load_stream(y + slot[j] * ys + v);
    }
  }
#pragma unroll
  for (int jv = 0; jv < VPT; ++jv) {
    const int32_t v = v0 + jv * THREADS;
    if (v >= nvec) continue;
    float acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = 0.0f;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (slot[j] < 0) continue;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        acc[2 * c] = __builtin_fmaf(w[j], bf16lo_to_f32(yv[jv][j][c]), acc[2 * c]);
        acc[2 * c + 1] = __builtin_fmaf(w[j], bf16hi_to_f32(yv[jv][j][c]), acc[2 * c + 1]);
      }
    }
    if (shared) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        acc[2 * c] = acc[2 * c] + bf16lo_to_f32(sv[jv][c]);
        acc[2 * c + 1] = acc[2 * c + 1] + bf16hi_to_f32(sv[jv][c]);
      }
    }
    u32x4 o;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      o[c] = f32_to_bf16_rne(acc[2 * c]) | (f32_to_bf16_rne(acc[2 * c + 1]) << 16);
    store_stream(o, out + (int64_t)t * nvec + v);
  }
}

// Quantised-transfer variant: expert rows are e4m3 codes with one fp32 scale
// per 128 channels (the dispatch's e4m3 format).  Each thread owns 16
// channels: per pair one 16-byte code load and one scale load (shared by the
// 8 lanes of a scale block), decode with the hardware e4m3 -> fp32
// conversion (exact), one fp32 multiply by the scale, then the same FMA chain,
// shared row and bf16 rounding as the bf16 combine.  One workgroup spans a
// whole row when it fits (up to 1024 threads), so each scale
// row is fetched by one compute unit instead of by one per chunk (measured:
// 66.4 -> 62.2 us at H = 7168 against 64-thread workgroups).
template <int KMAX>
__global__ __launch_bounds__(1024) void combine_fp8_kernel(
    const u32x4* __restrict__ y, int64_t ys, const float* __restrict__ yscale, int32_t nblk,
    int64_t cap, const int32_t* __restrict__ ids, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ send, const float* __restrict__ scales,
    const u32x4* __restrict__ shared, int64_t ss, int32_t ngroups, int32_t nchunks, int32_t k,
    int32_t E, u32x4* __restrict__ out, int32_t* status) {
  __shared__ int send_lds[kMaxExperts + 1];
  const int32_t t = blockIdx.x / nchunks;
  const int32_t chunk = blockIdx.x - t * nchunks;
  PairMeta meta;
  fetch_pair_meta(meta, t, k, ids, idx, scales);
  const int32_t g = chunk * (int32_t)blockDim.x + threadIdx.x;  // 16-channel group
  // The shared row does not depend on the routes: its loads go out first.
  u32x4 sh0 = {0u, 0u, 0u, 0u}, sh1 = {0u, 0u, 0u, 0u};
  if (shared && g < ngroups) {
    sh0 = load_stream(shared + (int64_t)t * ss + 2 * g);
    sh1 = load_stream(shared + (int64_t)t * ss + 2 * g + 1);
  }
  stage_send_any(send_lds, send, E);  // overlaps the fetches above
  int64_t slot[KMAX];
  float w[KMAX];
  resolve_routes<KMAX>(meta, send_lds, nullptr, k, E, cap, slot, w, status,
                       threadIdx.x < kWave && chunk == 0);

  if (g >= ngroups) return;  // no workgroup barrier follows
  u32x4 q[KMAX];
  float s[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (slot[j] < 0) continue;
    q[j] = load_stream(y + slot[j] * ys + g);
    s[j] = yscale[slot[j] * nblk + (g >> 3)];
  }

  float acc[16];
#pragma unroll
  for (int c = 0; c < 16; ++c) acc[c] = 0.0f;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (slot[j] < 0) continue;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)q[j][c], false);  // bytes 0, 1
      const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)q[j][c], true);   // bytes 2, 3
      const float d0 = lo[0] * s[j];
      const float d1 = lo[1] * s[j];
      const float d2 = hi[0] * s[j];
      const float d3 = hi[1] * s[j];
      acc[4 * c + 0] = __builtin_fmaf(w[j], d0, acc[4 * c + 0]);
      acc[4 * c + 1] = __builtin_fmaf(w[j], d1, acc[4 * c + 1]);
      acc[4 * c + 2] = __builtin_fmaf(w[j], d2, acc[4 * c + 2]);
      acc[4 * c + 3] = __builtin_fmaf(w[j], d3, acc[4 * c + 3]);
    }
  }
  if (shared) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      acc[2 * c] = acc[2 * c] + bf16lo_to_f32(sh0[c]);
      acc[2 * c + 1] = acc[2 * c + 1] + bf16hi_to_f32(sh0[c]);
      acc[8 + 2 * c] = acc[8 + 2 * c] + bf16lo_to_f32(sh1[c]);
      acc[8 + 2 * c + 1] = acc[8 + 2 * c + 1] + bf16hi_to_f32(sh1[c]);
    }
  }
  u32x4 o0, o1;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    o0[c] = f32_to_bf16_rne(acc[2 * c]) | (f32_to_bf16_rne(acc[2 * c + 1]) << 16);
    o1[c] = f32_to_bf16_rne(acc[8 + 2 * c]) | (f32_to_bf16_rne(acc[8 + 2 * c + 1]) << 16);
  }
  u32x4* dst = out + (int64_t)t * (2 * (int64_t)ngroups) + 2 * g;
  store_stream(o0, dst);
  store_stream(o1, dst + 1);
}

template <int THREADS, int VPT>
hipError_t launch_t(int kmax, dim3 grid, const u32x4* y, int64_t ys, int64_t cap,
                    const int32_t* ids, const int32_t* idx, const int32_t* send,
                    const float* scales, const u32x4* shared, int64_t ss, int32_t nvec,
                    int32_t nchunks, int32_t k, int32_t E, u32x4* out,
                    int32_t* status, hipStream_t stream) {
#define MOE_COMBINE(KM)                                                                   \
  launch_kernel(combine_kernel<THREADS, VPT, KM>, grid, THREADS, stream, y, ys, cap,       \
      ids, idx, send, scales, shared, ss, nvec, nchunks, k, E, out, status)
  switch (kmax) {
    case 2: MOE_COMBINE(2); break;
    case 4: MOE_COMBINE(4); break;
    case 8: MOE_COMBINE(8); break;
    default: MOE_COMBINE(16); break;
  }
#undef MOE_COMBINE
  return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(const void* y, int64_t y_stride, int64_t capacity_rows,
                          const int32_t* ids, const int32_t* expand_idx, const int32_t* send,
                          const float* scales, const void* shared, int64_t shared_stride,
                          int32_t bs, int32_t hidden, int32_t k, int32_t num_experts,
                          void* out, int32_t* status, hipStream_t stream) {
  constexpr int kThreads = MOE_COMBINE_THREADS;
  constexpr int kVpt = MOE_COMBINE_VPT;
  const int32_t nvec = hidden / 8;
  const int32_t nchunks = (nvec + kThreads * kVpt - 1) / (kThreads * kVpt);
  const int32_t n_items = bs * nchunks;
  const dim3 grid((uint32_t)n_items);
  const int kmax = k <= 2 ? 2 : k <= 4 ? 4 : k <= 8 ? 8 : 16;
  return launch_t<kThreads, kVpt>(kmax, grid, static_cast<const u32x4*>(y), y_stride / 8,
                                  capacity_rows, ids, expand_idx, send, scales,
                                  static_cast<const u32x4*>(shared), shared_stride / 8, nvec,
                                  nchunks, k, num_experts, static_cast<u32x4*>(out), status,
                                  stream);
}

}  // namespace moe

namespace moe {

hipError_t launch_combine_fp8(const void* y, int64_t y_stride, int64_t capacity_rows,
                              const float* y_scales, const int32_t* ids,
                              const int32_t* expand_idx, const int32_t* send,
                              const float* scales, const void* shared, int64_t shared_stride,
                              int32_t bs, int32_t hidden, int32_t k, int32_t num_experts,
                              void* out, int32_t* status, hipStream_t stream) {
  const int32_t ngroups = hidden / 16;
  const int32_t threads = ngroups <= 1024 ? (ngroups + kWave - 1) / kWave * kWave : 1024;
  const int32_t nchunks = (ngroups + threads - 1) / threads;
  const dim3 grid((uint32_t)(bs * nchunks));
  const u32x4* yv = static_cast<const u32x4*>(y);
  const u32x4* sv = static_cast<const u32x4*>(shared);
  u32x4* ov = static_cast<u32x4*>(out);
  const int64_t ys = y_stride / 16, ss = shared_stride / 8;
  const int32_t nblk = hidden / 128;
  const int kmax = k <= 2 ? 2 : k <= 4 ? 4 : k <= 8 ? 8 : 16;
  switch (kmax) {
    case 2:
      launch_kernel(combine_fp8_kernel<2>, grid, threads, stream,
          yv, ys, y_scales, nblk, capacity_rows, ids, expand_idx, send, scales, sv, ss, ngroups,
          nchunks, k, num_experts, ov, status);
      break;
    case 4:
      launch_kernel(combine_fp8_kernel<4>, grid, threads, stream,
          yv, ys, y_scales, nblk, capacity_rows, ids, expand_idx, send, scales, sv, ss, ngroups,
          nchunks, k, num_experts, ov, status);
      break;
    case 8:
      launch_kernel(combine_fp8_kernel<8>, grid, threads, stream,
          yv, ys, y_scales, nblk, capacity_rows, ids, expand_idx, send, scales, sv, ss, ngroups,
          nchunks, k, num_experts, ov, status);
      break;
    default:
      launch_kernel(combine_fp8_kernel<16>, grid, threads, stream,
          yv, ys, y_scales, nblk, capacity_rows, ids, expand_idx, send, scales, sv, ss, ngroups,
          nchunks, k, num_experts, ov, status);
      break;
  }
  return hipGetLastError();
}

}  // namespace moe
