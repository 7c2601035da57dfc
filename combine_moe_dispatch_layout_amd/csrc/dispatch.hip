// dispatch.hip -- scatter token rows into the expert-contiguous buffer
// (bf16 bit copy, or e4m3 quantisation with one fp32 scale per 128 channels
// fused into the scatter).  The combine on the npu_moe_distribute_combine page
// retraces exactly this path; row slot(t,j) = ep_send_counts[e] + expand_idx.
//
// Work split: one workgroup per item = (token, chunk of the row).  The
// workgroup stages ep_send_counts in LDS while lanes 0..K-1 fetch the token's
// ids and ranks, so the routes cost one memory round trip plus one LDS read.
// A row chunk is read once with 16-byte loads and written K times with
// 16-byte non-temporal stores (the dispatched rows are write-once streams).
// Every destination row is checked against capacity_rows before any store.
#include "moe_internal.h"

namespace moe {
namespace {

// LDS_INTS sizes the send-count array; a larger array than the counts need
// only serves to cap how many workgroups share a compute unit.
template <int THREADS, int VPT, int KMAX, int LDS_INTS>
__global__ __launch_bounds__(THREADS) void dispatch_bf16_kernel(
    const u32x4* __restrict__ x, int64_t xs, int32_t nvec, int32_t nchunks,
    const int32_t* __restrict__ ids, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ send, int32_t k, int32_t E, u32x4* __restrict__ out, int64_t os,
    int64_t cap, int32_t* status) {
  static_assert(LDS_INTS >= kMaxExperts + 1, "send counts must fit");
  __shared__ int send_lds[LDS_INTS];
  const int32_t t = blockIdx.x / nchunks;
  const int32_t chunk = blockIdx.x - t * nchunks;
  PairMeta meta;
  fetch_pair_meta(meta, t, k, ids, idx, nullptr);
  const int32_t v0 = chunk * (THREADS * VPT) + threadIdx.x;
  const u32x4* src = x + (int64_t)t * xs;
  u32x4 r[VPT];
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    const int32_t v = v0 + j * THREADS;
    if (v < nvec) r[j] = src[v];
  }
  stage_send(send_lds, send, E);  // overlaps the loads above
  int64_t slot[KMAX];
  float unused_w[KMAX];
  resolve_routes<KMAX>(meta, send_lds, k, E, cap, slot, unused_w, status,
                       threadIdx.x < kWave && chunk == 0);
#pragma unroll
  for (int jj = 0; jj < KMAX; ++jj) {
    if (slot[jj] < 0) continue;
    u32x4* dst = out + slot[jj] * os;
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int32_t v = v0 + j * THREADS;
      if (v < nvec) store_stream(r[j], dst + v);
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
  __shared__ int send_lds[kMaxExperts + 1];
  const int32_t t = blockIdx.x / nchunks;
  const int32_t chunk = blockIdx.x - t * nchunks;
  PairMeta meta;
  fetch_pair_meta(meta, t, k, ids, idx, nullptr);

  const int32_t g = chunk * THREADS + threadIdx.x;  // 16-channel group within the row
  const bool active = g < ngroups;
  u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
  if (active) {
    const u32x4* src = x + (int64_t)t * xs + 2 * (int64_t)g;
    a = src[0];
    b = src[1];
  }
  stage_send(send_lds, send, E);  // overlaps the loads above
  int64_t slot[KMAX];
  float unused_w[KMAX];
  resolve_routes<KMAX>(meta, send_lds, k, E, cap, slot, unused_w, status,
                       threadIdx.x < kWave && chunk == 0);

  float s;
  const u32x4 codes = quantize16_e4m3(a, b, s);

  // Code rows are written with streaming stores (each wave covers whole
  // lines).  A wave holds only 32 bytes of a scale row, so scale stores stay
  // ordinary cached stores: L2 merges the pieces of a line before it is
  // written back, where streaming partial-line writes would each reach HBM
  // (measured on the 4096-token e4m3 dispatch with the token rows read from
  // HBM: 71.0-71.5 us with streaming scale stores, 64.1-64.2 us with these).
  const bool writes_scale = active && (g & 7) == 0;
#pragma unroll
  for (int jj = 0; jj < KMAX; ++jj) {
    if (slot[jj] < 0) continue;
    if (active) store_stream(codes, out + slot[jj] * os + g);
    if (writes_scale) scales[slot[jj] * nblk + (g >> 3)] = s;
  }
}

int kmax_for(int32_t k) { return k <= 2 ? 2 : k <= 4 ? 4 : k <= 8 ? 8 : 16; }

// Launch shape of the bf16 scatter.  With the token rows already in the
// Infinity Cache (read ahead by the layout launches), the scatter is bound
// by its row writes alone, and HBM takes them faster from fewer waves in
// flight, which write a narrower window of destination rows: 64-thread
// workgroups holding 19 KB of LDS each, so that at most 8 share a compute
// unit (2 waves per SIMD).  Rows that still come from HBM need the latency
// hiding of full occupancy, so they keep 128-thread workgroups with only
// the send counts in LDS.
template <int THREADS, int LDS_INTS>
hipError_t launch_bf16_shape(const void* x, int64_t x_stride, int32_t bs, int32_t hidden,
                             const int32_t* ids, const int32_t* expand_idx, const int32_t* send,
                             int32_t k, int32_t num_experts, void* expand_x,
                             int64_t expand_x_stride, int64_t capacity_rows, int32_t* status,
                             hipStream_t stream) {
  constexpr int kVpt = MOE_DISPATCH_VPT;
  const int32_t nvec = hidden / 8;  // 16-byte vectors per row
  const int32_t nchunks = (nvec + THREADS * kVpt - 1) / (THREADS * kVpt);
  const int32_t n_items = bs * nchunks;
  const dim3 grid((uint32_t)n_items);
  const u32x4* xv = static_cast<const u32x4*>(x);
  u32x4* ov = static_cast<u32x4*>(expand_x);
  const int64_t xs = x_stride / 8, os = expand_x_stride / 8;
  switch (kmax_for(k)) {
    case 2:
      launch_kernel(dispatch_bf16_kernel<THREADS, kVpt, 2, LDS_INTS>, grid, THREADS, stream,
          xv, xs, nvec, nchunks, ids, expand_idx, send, k, num_experts, ov, os,
          capacity_rows, status);
      break;
    case 4:
      launch_kernel(dispatch_bf16_kernel<THREADS, kVpt, 4, LDS_INTS>, grid, THREADS, stream,
          xv, xs, nvec, nchunks, ids, expand_idx, send, k, num_experts, ov, os,
          capacity_rows, status);
      break;
    case 8:
      launch_kernel(dispatch_bf16_kernel<THREADS, kVpt, 8, LDS_INTS>, grid, THREADS, stream,
          xv, xs, nvec, nchunks, ids, expand_idx, send, k, num_experts, ov, os,
          capacity_rows, status);
      break;
    default:
      launch_kernel(dispatch_bf16_kernel<THREADS, kVpt, 16, LDS_INTS>, grid, THREADS, stream,
          xv, xs, nvec, nchunks, ids, expand_idx, send, k, num_experts, ov, os,
          capacity_rows, status);
      break;
  }
  return hipGetLastError();
}

constexpr int kCachedRowsThreads = 64;
constexpr int kCachedRowsLdsInts = 19456 / 4;  // 8 workgroups in a compute unit's 160 KB

}  // namespace

hipError_t launch_dispatch_bf16(const void* x, int64_t x_stride, int32_t bs, int32_t hidden,
                                const int32_t* ids, const int32_t* expand_idx,
                                const int32_t* send, int32_t k, int32_t num_experts,
                                void* expand_x, int64_t expand_x_stride, int64_t capacity_rows,
                                int32_t* status, hipStream_t stream, bool rows_cached) {
  if (rows_cached)
    return launch_bf16_shape<kCachedRowsThreads, kCachedRowsLdsInts>(
        x, x_stride, bs, hidden, ids, expand_idx, send, k, num_experts, expand_x,
        expand_x_stride, capacity_rows, status, stream);
  return launch_bf16_shape<MOE_DISPATCH_THREADS, kMaxExperts + 1>(
      x, x_stride, bs, hidden, ids, expand_idx, send, k, num_experts, expand_x,
      expand_x_stride, capacity_rows, status, stream);
}

hipError_t launch_dispatch_fp8(const void* x, int64_t x_stride, int32_t bs, int32_t hidden,
                               const int32_t* ids, const int32_t* expand_idx,
                               const int32_t* send, int32_t k, int32_t num_experts,
                               void* expand_x, int64_t expand_x_stride, int64_t capacity_rows,
                               float* quant_scales, int32_t* status, hipStream_t stream) {
  constexpr int kThreads = MOE_FP8_THREADS;
  const int32_t ngroups = hidden / 16;
  const int32_t nchunks = (ngroups + kThreads - 1) / kThreads;
  const int32_t n_items = bs * nchunks;
  const dim3 grid((uint32_t)n_items);
  const u32x4* xv = static_cast<const u32x4*>(x);
  u32x4* ov = static_cast<u32x4*>(expand_x);
  const int64_t xs = x_stride / 8, os = expand_x_stride / 16;
  const int32_t nblk = hidden / 128;
  switch (kmax_for(k)) {
    case 2:
      launch_kernel(dispatch_fp8_kernel<kThreads, 2>, grid, kThreads, stream,
          xv, xs, ngroups, nchunks, ids, expand_idx, send, k, num_experts, ov, os,
          quant_scales, nblk, capacity_rows, status);
      break;
    case 4:
      launch_kernel(dispatch_fp8_kernel<kThreads, 4>, grid, kThreads, stream,
          xv, xs, ngroups, nchunks, ids, expand_idx, send, k, num_experts, ov, os,
          quant_scales, nblk, capacity_rows, status);
      break;
    case 8:
      launch_kernel(dispatch_fp8_kernel<kThreads, 8>, grid, kThreads, stream,
          xv, xs, ngroups, nchunks, ids, expand_idx, send, k, num_experts, ov, os,
          quant_scales, nblk, capacity_rows, status);
      break;
    default:
      launch_kernel(dispatch_fp8_kernel<kThreads, 16>, grid, kThreads, stream,
          xv, xs, ngroups, nchunks, ids, expand_idx, send, k, num_experts, ov, os,
          quant_scales, nblk, capacity_rows, status);
      break;
  }
  return hipGetLastError();
}

}  // namespace moe
