// fused.hip -- layout and bf16 scatter in one launch for small batches
// (decode-sized: at most kFusedMaxPairs (token, expert) pairs).
//
// At this size the layout of the npu_moe_distribute_combine page's
// expert_ids / expand_idx / ep_send_counts triple (with the TEMPO summary's
// 128-row M-tile padding, section 1) is cheap enough for every workgroup of
// the scatter to derive it by itself, so no workgroup waits for another and
// the separate layout launch and its latency disappear:
//   - the workgroup issues the load of its row chunk first (it does not
//     depend on the layout), then loads all ids once into LDS;
//   - two LDS histograms count every expert's pairs and the pairs of the
//     tokens before its own token;
//   - a workgroup-wide exclusive scan of the padded counts gives the
//     segment offsets;
//   - lane j < K of each wave forms pair (t, j)'s rank (pairs of earlier
//     tokens on the same expert, plus earlier repeats of that expert in the
//     row) and its destination row, which are broadcast through the wave.
// Workgroup 0 also writes expert_counts, ep_send_counts and the status word
// (out-of-range ids, repeated ids within a row, rows beyond capacity), and
// the first-chunk workgroup of every token writes that token's expand_idx,
// so the outputs equal those of the separate layout and scatter calls.
#include "moe_internal.h"

namespace moe {
namespace {

template <int THREADS, int KMAX>
__global__ __launch_bounds__(THREADS) void dispatch_fused_bf16_kernel(
    const u32x4* __restrict__ x, int64_t xs, int32_t nvec, int32_t nchunks,
    const int32_t* __restrict__ ids, int32_t n_pairs, int32_t k, int32_t E, int32_t align,
    int32_t* __restrict__ counts, int32_t* __restrict__ send, int32_t* __restrict__ expand_idx,
    int32_t* __restrict__ status, u32x4* __restrict__ out, int64_t os, int64_t cap) {
  constexpr int kIdsPerThread = kFusedMaxPairs / THREADS;
  constexpr int kBins = kMaxExperts / THREADS;  // experts per thread in the scan
  constexpr int kWaves = THREADS / kWave;
  static_assert(kFusedMaxPairs % THREADS == 0 && kMaxExperts % THREADS == 0, "shape");
  __shared__ int ids_lds[kFusedMaxPairs];
  __shared__ int hist[kMaxExperts];
  __shared__ int before[kMaxExperts];
  __shared__ int send_lds[kMaxExperts + 1];
  __shared__ int wave_tot[kWaves];
  __shared__ int flags_lds;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int32_t t = blockIdx.x / nchunks;
  const int32_t chunk = blockIdx.x - t * nchunks;
  const int32_t v = chunk * THREADS + tid;

  // The row chunk and all ids: every load is issued before the first wait.
  u32x4 row = {0u, 0u, 0u, 0u};
  if (v < nvec) row = x[(int64_t)t * xs + v];
  int idv[kIdsPerThread];
#pragma unroll
  for (int s = 0; s < kIdsPerThread; ++s) {
    const int p = s * THREADS + tid;
    idv[s] = (p < n_pairs) ? ids[p] : -1;
  }
  for (int e = tid; e < E; e += THREADS) {
    hist[e] = 0;
    before[e] = 0;
  }
  if (tid == 0) flags_lds = 0;
  __syncthreads();

  const int first = t * k;  // this token's first pair
  int fl = 0;
#pragma unroll
  for (int s = 0; s < kIdsPerThread; ++s) {
    const int p = s * THREADS + tid;
    if (p < n_pairs) {
      const int e = idv[s];
      ids_lds[p] = e;
      if (e >= 0 && e < E) {
        atomicAdd(&hist[e], 1);
        if (p < first) atomicAdd(&before[e], 1);
      } else {
        fl |= MOE_FLAG_ID_RANGE;
      }
    }
  }
  __syncthreads();

  // Exclusive scan of the padded counts; thread i owns experts
  // [i*kBins, (i+1)*kBins).
  int padded[kBins];
  int own = 0;
#pragma unroll
  for (int b = 0; b < kBins; ++b) {
    const int e = tid * kBins + b;
    const int c = (e < E) ? hist[e] : 0;
    padded[b] = (c + align - 1) & ~(align - 1);
    own += padded[b];
  }
  int incl = own;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int o = __shfl_up(incl, d, kWave);
    if (lane >= d) incl += o;
  }
  if (lane == kWave - 1) wave_tot[wave] = incl;
  __syncthreads();
  int run = incl - own;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) run += (w < wave) ? wave_tot[w] : 0;
#pragma unroll
  for (int b = 0; b < kBins; ++b) {
    const int e = tid * kBins + b;
    if (e < E) send_lds[e] = run;
    run += padded[b];
  }
  if (tid == THREADS - 1) send_lds[E] = run;  // the last thread's running sum is the total
  __syncthreads();

  // Routes of token t, formed by lanes 0..k-1 of every wave.
  int my_rank = -1;
  int64_t my_slot = -1;
  if (lane < k) {
    const int e = ids_lds[first + lane];
    if (e >= 0 && e < E) {
      int repeats = 0;
      for (int j = 0; j < lane; ++j) repeats += (ids_lds[first + j] == e) ? 1 : 0;
      my_rank = before[e] + repeats;
      const int64_t s = (int64_t)send_lds[e] + my_rank;
      if (s < cap) my_slot = s;
    }
  }
  const int32_t lo = (int32_t)(my_slot & 0xFFFFFFFF);
  const int32_t hi = (int32_t)(my_slot >> 32);
  int64_t slot[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    const uint32_t l = (uint32_t)__builtin_amdgcn_readlane(lo, j);
    const int32_t h = __builtin_amdgcn_readlane(hi, j);
    slot[j] = (j < k) ? (int64_t)(((uint64_t)(uint32_t)h << 32) | l) : -1;
  }

  if (v < nvec) {
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (slot[j] >= 0) store_stream(row, out + slot[j] * os + v);
  }
  if (chunk == 0 && wave == 0 && lane < k) expand_idx[first + lane] = my_rank;

  if (blockIdx.x == 0) {  // workgroup-uniform
    for (int e = tid; e < E; e += THREADS) {
      const int c = hist[e];
      counts[e] = c;
      send[e] = send_lds[e];
      // the highest rank of expert e is c - 1
      if (c > 0 && (int64_t)send_lds[e] + c - 1 >= cap) fl |= MOE_FLAG_GUARD;
    }
    if (tid == 0) send[E] = send_lds[E];
    for (int tt = tid; tt * k < n_pairs; tt += THREADS) {
      for (int a = 1; a < k; ++a) {
        const int ea = ids_lds[tt * k + a];
        for (int b = 0; b < a; ++b)
          if (ea == ids_lds[tt * k + b] && ea >= 0 && ea < E) fl |= MOE_FLAG_DUP_ID;
      }
    }
    if (fl) atomicOr(&flags_lds, fl);
    __syncthreads();
    if (tid == 0 && status) *status = flags_lds;
  }
}

}  // namespace

hipError_t launch_dispatch_fused_bf16(const void* x, int64_t x_stride, int32_t bs,
                                      int32_t hidden, const int32_t* ids, int32_t k,
                                      int32_t num_experts, int32_t align, int32_t* counts,
                                      int32_t* send, int32_t* expand_idx, int32_t* status,
                                      void* expand_x, int64_t expand_x_stride,
                                      int64_t capacity_rows, hipStream_t stream) {
  constexpr int kThreads = MOE_DISPATCH_THREADS;
  const int32_t nvec = hidden / 8;
  const int32_t nchunks = (nvec + kThreads - 1) / kThreads;
  const dim3 grid((uint32_t)(bs * nchunks));
  const u32x4* xv = static_cast<const u32x4*>(x);
  u32x4* ov = static_cast<u32x4*>(expand_x);
  const int64_t xs = x_stride / 8, os = expand_x_stride / 8;
  const int32_t n = bs * k;
  const int kmax = k <= 2 ? 2 : k <= 4 ? 4 : k <= 8 ? 8 : 16;
  switch (kmax) {
    case 2:
      dispatch_fused_bf16_kernel<kThreads, 2><<<grid, kThreads, 0, stream>>>(
          xv, xs, nvec, nchunks, ids, n, k, num_experts, align, counts, send, expand_idx, status,
          ov, os, capacity_rows);
      break;
    case 4:
      dispatch_fused_bf16_kernel<kThreads, 4><<<grid, kThreads, 0, stream>>>(
          xv, xs, nvec, nchunks, ids, n, k, num_experts, align, counts, send, expand_idx, status,
          ov, os, capacity_rows);
      break;
    case 8:
      dispatch_fused_bf16_kernel<kThreads, 8><<<grid, kThreads, 0, stream>>>(
          xv, xs, nvec, nchunks, ids, n, k, num_experts, align, counts, send, expand_idx, status,
          ov, os, capacity_rows);
      break;
    default:
      dispatch_fused_bf16_kernel<kThreads, 16><<<grid, kThreads, 0, stream>>>(
          xv, xs, nvec, nchunks, ids, n, k, num_experts, align, counts, send, expand_idx, status,
          ov, os, capacity_rows);
      break;
  }
  return hipGetLastError();
}

}  // namespace moe
