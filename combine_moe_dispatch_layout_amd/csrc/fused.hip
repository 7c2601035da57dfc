// fused.hip -- layout and scatter (bf16, or e4m3 with per-128-channel
// scales) in one launch for small batches (decode-sized: at most
// kFusedMaxPairs (token, expert) pairs).
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

// LDS state of the layout each workgroup derives.
struct FusedLds {
  int ids[kFusedMaxPairs];
  int hist[kMaxExperts];    // pairs per expert
  int before[kMaxExperts];  // pairs per expert among the tokens before this one
  int send[kMaxExperts + 1];
  int wave_tot[16];
  int flags;
};

// Derives the layout in LDS and returns token t's destination rows in
// slot[] (-1: pair skipped), identical in every wave.  The caller issues its
// row loads first so that they overlap this.  Workgroup 0 writes counts,
// offsets and status; the first-chunk workgroup of token t writes t's ranks.
template <int THREADS, int KMAX>
__device__ __forceinline__ void fused_layout(FusedLds& L, const int32_t* __restrict__ ids,
                                             int32_t n_pairs, int32_t k, int32_t E,
                                             int32_t align, int32_t t, int32_t chunk, int64_t cap,
                                             int32_t* __restrict__ counts,
                                             int32_t* __restrict__ send,
                                             int32_t* __restrict__ expand_idx,
                                             int32_t* __restrict__ status, int64_t (&slot)[KMAX]) {
  constexpr int kIdsPerThread = kFusedMaxPairs / THREADS;
  constexpr int kBins = kMaxExperts / THREADS;  // experts per thread in the scan
  constexpr int kWaves = THREADS / kWave;
  static_assert(kFusedMaxPairs % THREADS == 0 && kMaxExperts % THREADS == 0, "shape");
  static_assert(kWaves <= 16, "wave totals");
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;

  int idv[kIdsPerThread];
#pragma unroll
  for (int s = 0; s < kIdsPerThread; ++s) {
    const int p = s * THREADS + tid;
    idv[s] = (p < n_pairs) ? ids[p] : -1;
  }
  for (int e = tid; e < E; e += THREADS) {
    L.hist[e] = 0;
    L.before[e] = 0;
  }
  if (tid == 0) L.flags = 0;
  __syncthreads();

  const int first = t * k;  // this token's first pair
  int fl = 0;
#pragma unroll
  for (int s = 0; s < kIdsPerThread; ++s) {
    const int p = s * THREADS + tid;
    if (p < n_pairs) {
      const int e = idv[s];
      L.ids[p] = e;
      if (e >= 0 && e < E) {
        atomicAdd(&L.hist[e], 1);
        if (p < first) atomicAdd(&L.before[e], 1);
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
    const int c = (e < E) ? L.hist[e] : 0;
    padded[b] = (c + align - 1) & ~(align - 1);
    own += padded[b];
  }
  int incl = own;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int o = __shfl_up(incl, d, kWave);
    if (lane >= d) incl += o;
  }
  if (lane == kWave - 1) L.wave_tot[wave] = incl;
  __syncthreads();
  int run = incl - own;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) run += (w < wave) ? L.wave_tot[w] : 0;
#pragma unroll
  for (int b = 0; b < kBins; ++b) {
    const int e = tid * kBins + b;
    if (e < E) L.send[e] = run;
    run += padded[b];
  }
  if (tid == THREADS - 1) L.send[E] = run;  // the last thread's running sum is the total
  __syncthreads();

  // Routes of token t, formed by lanes 0..k-1 of every wave.
  int my_rank = -1;
  int64_t my_slot = -1;
  if (lane < k) {
    const int e = L.ids[first + lane];
    if (e >= 0 && e < E) {
      int repeats = 0;
      for (int j = 0; j < lane; ++j) repeats += (L.ids[first + j] == e) ? 1 : 0;
      my_rank = L.before[e] + repeats;
      const int64_t s = (int64_t)L.send[e] + my_rank;
      if (s < cap) my_slot = s;
    }
  }
  const int32_t lo = (int32_t)(my_slot & 0xFFFFFFFF);
  const int32_t hi = (int32_t)(my_slot >> 32);
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    const uint32_t l = (uint32_t)__builtin_amdgcn_readlane(lo, j);
    const int32_t h = __builtin_amdgcn_readlane(hi, j);
    slot[j] = (j < k) ? (int64_t)(((uint64_t)(uint32_t)h << 32) | l) : -1;
  }
  if (chunk == 0 && wave == 0 && lane < k) expand_idx[first + lane] = my_rank;

  if (blockIdx.x == 0) {  // workgroup-uniform
    for (int e = tid; e < E; e += THREADS) {
      const int c = L.hist[e];
      counts[e] = c;
      send[e] = L.send[e];
      // the highest rank of expert e is c - 1
      if (c > 0 && (int64_t)L.send[e] + c - 1 >= cap) fl |= MOE_FLAG_GUARD;
    }
    if (tid == 0) send[E] = L.send[E];
    for (int tt = tid; tt * k < n_pairs; tt += THREADS) {
      for (int a = 1; a < k; ++a) {
        const int ea = L.ids[tt * k + a];
        for (int b = 0; b < a; ++b)
          if (ea == L.ids[tt * k + b] && ea >= 0 && ea < E) fl |= MOE_FLAG_DUP_ID;
      }
    }
    if (fl) atomicOr(&L.flags, fl);
    __syncthreads();
    if (tid == 0 && status) *status = L.flags;
  }
}

// bf16: one workgroup per (token, THREADS 16-byte vectors of the row).
template <int THREADS, int KMAX>
__global__ __launch_bounds__(THREADS) void dispatch_fused_bf16_kernel(
    const u32x4* __restrict__ x, int64_t xs, int32_t nvec, int32_t nchunks,
    const int32_t* __restrict__ ids, int32_t n_pairs, int32_t k, int32_t E, int32_t align,
    int32_t* __restrict__ counts, int32_t* __restrict__ send, int32_t* __restrict__ expand_idx,
    int32_t* __restrict__ status, u32x4* __restrict__ out, int64_t os, int64_t cap) {
  __shared__ FusedLds lds;
  const int32_t t = blockIdx.x / nchunks;
  const int32_t chunk = blockIdx.x - t * nchunks;
  const int32_t v = chunk * THREADS + threadIdx.x;
  u32x4 row = {0u, 0u, 0u, 0u};
  if (v < nvec) row = x[(int64_t)t * xs + v];  // independent of the layout: issued first
  int64_t slot[KMAX];
  fused_layout<THREADS, KMAX>(lds, ids, n_pairs, k, E, align, t, chunk, cap, counts, send,
                              expand_idx, status, slot);
  if (v < nvec) {
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (slot[j] >= 0) store_stream(row, out + slot[j] * os + v);
  }
}

// e4m3: one workgroup per (token, THREADS 16-channel groups of the row),
// quantised as in the separate e4m3 dispatch; scale stores stay ordinary
// cached stores so that L2 merges a row's scale pieces.
template <int THREADS, int KMAX>
__global__ __launch_bounds__(THREADS) void dispatch_fused_fp8_kernel(
    const u32x4* __restrict__ x, int64_t xs, int32_t ngroups, int32_t nchunks,
    const int32_t* __restrict__ ids, int32_t n_pairs, int32_t k, int32_t E, int32_t align,
    int32_t* __restrict__ counts, int32_t* __restrict__ send, int32_t* __restrict__ expand_idx,
    int32_t* __restrict__ status, u32x4* __restrict__ out, int64_t os,
    float* __restrict__ scales, int32_t nblk, int64_t cap) {
  __shared__ FusedLds lds;
  const int32_t t = blockIdx.x / nchunks;
  const int32_t chunk = blockIdx.x - t * nchunks;
  const int32_t g = chunk * THREADS + threadIdx.x;  // 16-channel group within the row
  const bool active = g < ngroups;
  u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
  if (active) {
    const u32x4* src = x + (int64_t)t * xs + 2 * (int64_t)g;
    a = src[0];
    b = src[1];
  }
  int64_t slot[KMAX];
  fused_layout<THREADS, KMAX>(lds, ids, n_pairs, k, E, align, t, chunk, cap, counts, send,
                              expand_idx, status, slot);
  float s;
  const u32x4 codes = quantize16_e4m3(a, b, s);
  const bool writes_scale = active && (g & 7) == 0;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (slot[j] < 0) continue;
    if (active) store_stream(codes, out + slot[j] * os + g);
    if (writes_scale) scales[slot[j] * nblk + (g >> 3)] = s;
  }
}

int kmax_of(int32_t k) { return k <= 2 ? 2 : k <= 4 ? 4 : k <= 8 ? 8 : 16; }

}  // namespace

hipError_t launch_dispatch_fused_bf16(const void* x, int64_t x_stride, int32_t bs,
                                      int32_t hidden, const int32_t* ids, int32_t k,
                                      int32_t num_experts, int32_t align, int32_t* counts,
                                      int32_t* send, int32_t* expand_idx, int32_t* status,
                                      void* expand_x, int64_t expand_x_stride,
                                      int64_t capacity_rows, hipStream_t stream) {
  constexpr int kThreads = MOE_FUSED_THREADS;
  const int32_t nvec = hidden / 8;
  const int32_t nchunks = (nvec + kThreads - 1) / kThreads;
  const dim3 grid((uint32_t)(bs * nchunks));
  const u32x4* xv = static_cast<const u32x4*>(x);
  u32x4* ov = static_cast<u32x4*>(expand_x);
  const int64_t xs = x_stride / 8, os = expand_x_stride / 8;
  const int32_t n = bs * k;
#define MOE_FUSED_BF16(KM)                                                                    \
  launch_kernel(dispatch_fused_bf16_kernel<kThreads, KM>, grid, kThreads, stream,             \
      xv, xs, nvec, nchunks, ids, n, k, num_experts, align, counts, send, expand_idx, status, \
      ov, os, capacity_rows)
  switch (kmax_of(k)) {
    case 2: MOE_FUSED_BF16(2); break;
    case 4: MOE_FUSED_BF16(4); break;
    case 8: MOE_FUSED_BF16(8); break;
    default: MOE_FUSED_BF16(16); break;
  }
#undef MOE_FUSED_BF16
  return hipGetLastError();
}

hipError_t launch_dispatch_fused_fp8(const void* x, int64_t x_stride, int32_t bs,
                                     int32_t hidden, const int32_t* ids, int32_t k,
                                     int32_t num_experts, int32_t align, int32_t* counts,
                                     int32_t* send, int32_t* expand_idx, int32_t* status,
                                     void* expand_x, int64_t expand_x_stride,
                                     int64_t capacity_rows, float* quant_scales,
                                     hipStream_t stream) {
  constexpr int kThreads = MOE_FP8_THREADS;
  const int32_t ngroups = hidden / 16;
  const int32_t nchunks = (ngroups + kThreads - 1) / kThreads;
  const dim3 grid((uint32_t)(bs * nchunks));
  const u32x4* xv = static_cast<const u32x4*>(x);
  u32x4* ov = static_cast<u32x4*>(expand_x);
  const int64_t xs = x_stride / 8, os = expand_x_stride / 16;
  const int32_t nblk = hidden / 128;
  const int32_t n = bs * k;
#define MOE_FUSED_FP8(KM)                                                                     \
  launch_kernel(dispatch_fused_fp8_kernel<kThreads, KM>, grid, kThreads, stream,              \
      xv, xs, ngroups, nchunks, ids, n, k, num_experts, align, counts, send, expand_idx,      \
      status, ov, os, quant_scales, nblk, capacity_rows)
  switch (kmax_of(k)) {
    case 2: MOE_FUSED_FP8(2); break;
    case 4: MOE_FUSED_FP8(4); break;
    case 8: MOE_FUSED_FP8(8); break;
    default: MOE_FUSED_FP8(16); break;
  }
#undef MOE_FUSED_FP8
  return hipGetLastError();
}

}  // namespace moe
