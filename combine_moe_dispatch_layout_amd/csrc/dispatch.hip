// dispatch.hip -- scatter token rows into the expert-contiguous buffer
// (bf16 bit copy, or e4m3 quantisation with one fp32 scale per 128 channels
// fused into the scatter).  The combine on the npu_moe_distribute_combine page
// retraces exactly this path; row slot(t,j) = ep_send_counts[e] + expand_idx.
//
// Work split: one workgroup per item = (token, chunk of the row).  The
// workgroup stages ep_send_counts in LDS while lanes 0..K-1 fetch the token's
// ids and ranks, so the routes cost one memory round trip plus one LDS read
// (in large grids of rows from HBM the staging is deliberately slower; see
// Staging below).
// A row chunk is read once with 16-byte loads and written K times with
// 16-byte non-temporal stores (the dispatched rows are write-once streams).
// Every destination row is checked against capacity_rows before any store.
#include "moe_internal.h"

namespace moe {
namespace {

// The routes' offset tables, staged in LDS in two steps (load, then store)
// around the row loads: the send counts, and with deferred ranks also the
// column prefix of the ranking workgroup that holds token t (kBase ints
// into the LDS area, which holds at least kInts ints).
template <int THREADS, bool DEFER>
struct RouteTables {
  using Send = StagedSend<THREADS>;
  using Base = StagedInts<THREADS, (DEFER ? kMaxExperts : 1)>;
  static constexpr int kBase = Send::kSlots;
  static constexpr int kInts = Send::kSlots + (DEFER ? Base::kSlots : 0);
  Send send;
  Base base;
  __device__ __forceinline__ void load(const int32_t* __restrict__ send_counts,
                                       const DeferredRanks& dr, int32_t t, int32_t E) {
    send.load(send_counts, E + 1);
    if (DEFER) base.load(dr.base + (int64_t)(t / dr.tokens_per_block) * E, E);
  }
  // Writes the tables and synchronises; returns the column prefix table
  // (nullptr without deferred ranks).
  __device__ __forceinline__ const int* store(int* lds) const {
    send.store(lds);
    if (DEFER) base.store(lds + kBase);
    __syncthreads();
    return DEFER ? lds + kBase : nullptr;
  }
  // The same tables, each thread staging its entries one load at a time
  // (a round trip per entry; see Staging::kRowsFirstSerial).
  __device__ __forceinline__ static const int* stage_serial(
      int* lds, const int32_t* __restrict__ send_counts, const DeferredRanks& dr, int32_t t,
      int32_t E) {
    if (DEFER) {
      const int32_t* row = dr.base + (int64_t)(t / dr.tokens_per_block) * E;
      for (int e = threadIdx.x; e < E; e += THREADS) lds[kBase + e] = row[e];
    }
    for (int e = threadIdx.x; e <= E; e += THREADS) lds[e] = send_counts[e];
    __syncthreads();
    return DEFER ? lds + kBase : nullptr;
  }
};

// Order of a workgroup's loads before its stores, chosen per launch:
//  - kTablesFirst: the tables' loads, then the row's (rows already in the
//    Infinity Cache); staging is one round trip and the routes need not wait
//    for the row;
//  - kRowsFirst: the row's loads (from HBM), then the tables' in one round
//    trip that overlaps the row's latency (latency-bound, decode-sized
//    grids);
//  - kRowsFirstSerial: the row's loads, then the tables staged one load at a
//    time per thread.  The longer workgroup life leaves fewer writes in
//    flight, which HBM takes faster in bandwidth-bound grids (measured on the
//    16384-token, E = 512 line: 374 us against 401 us batched, with the cap
//    of kUncachedPerCu workgroups per compute unit).
enum class Staging { kTablesFirst, kRowsFirst, kRowsFirstSerial };

// With deferred ranks, the first-chunk workgroup of token t writes the
// token's final expand_idx (rank within the workgroup + column prefix).
template <bool DEFER>
__device__ __forceinline__ void write_deferred(const PairMeta& m, const int* base_lds,
                                               const DeferredRanks& dr, int32_t t, int32_t k,
                                               int32_t E, bool first_chunk) {
  if (!DEFER || !first_chunk || threadIdx.x >= (unsigned)k) return;
  const bool ok = m.r >= 0 && m.e >= 0 && m.e < E;
  dr.expand_idx[(int64_t)t * k + threadIdx.x] = ok ? base_lds[m.e] + m.r : -1;
}

// LDS_INTS sizes the offset tables; a larger array than they need only
// serves to cap how many workgroups share a compute unit.
template <int THREADS, int VPT, int KMAX, int LDS_INTS, bool DEFER, Staging ORDER>
__global__ __launch_bounds__(THREADS) void dispatch_bf16_kernel(
    const u32x4* x, int64_t xs, int32_t nvec, int32_t nchunks,
    const int32_t* __restrict__ ids, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ send, int32_t k, int32_t E, u32x4* __restrict__ out, int64_t os,
    int64_t cap, int32_t* status, DeferredRanks dr) {
  static_assert(LDS_INTS >= RouteTables<THREADS, DEFER>::kInts, "tables must fit");
  __shared__ int lds[LDS_INTS];
  const int32_t t = blockIdx.x / nchunks;
  const int32_t chunk = blockIdx.x - t * nchunks;
  PairMeta meta;
  fetch_pair_meta(meta, t, k, ids, idx, nullptr);
  // (A lane past the row end repeats the last vector and stores nothing, so
  // the row loads need no branch.)
  const int32_t v0 = chunk * (THREADS * VPT) + threadIdx.x;
  const u32x4* src = x + (int64_t)t * xs;
  u32x4 r[VPT];
  RouteTables<THREADS, DEFER> tables;
  const int* base_lds;
  if (ORDER == Staging::kRowsFirstSerial) {
#pragma unroll
    for (int j = 0; j < VPT; ++j) r[j] = src[min(v0 + j * THREADS, nvec - 1)];
    base_lds = RouteTables<THREADS, DEFER>::stage_serial(lds, send, dr, t, E);
  } else {
    if (ORDER == Staging::kRowsFirst) {
#pragma unroll
      for (int j = 0; j < VPT; ++j) r[j] = src[min(v0 + j * THREADS, nvec - 1)];
      tables.load(send, dr, t, E);
    } else {
      tables.load(send, dr, t, E);
#pragma unroll
      for (int j = 0; j < VPT; ++j) r[j] = src[min(v0 + j * THREADS, nvec - 1)];
    }
    keep_order();
    base_lds = tables.store(lds);
  }
  int64_t slot[KMAX];
  float unused_w[KMAX];
  resolve_routes<KMAX>(meta, lds, base_lds, k, E, cap, slot, unused_w, status,
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
  write_deferred<DEFER>(meta, base_lds, dr, t, k, E, chunk == 0);
}

// Each thread owns 16 consecutive channels (two 16-byte loads of bf16, one
// 16-byte store of e4m3 codes); 8 neighbouring lanes form one 128-channel
// scale block and combine their maxima with cross-lane exchanges.
template <int THREADS, int KMAX, bool DEFER, int LDS_INTS>
__global__ __launch_bounds__(THREADS) void dispatch_fp8_kernel(
    const u32x4* x, int64_t xs, int32_t ngroups, int32_t nchunks,
    const int32_t* __restrict__ ids, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ send, int32_t k, int32_t E, u32x4* __restrict__ out, int64_t os,
    float* __restrict__ scales, int32_t nblk, int64_t cap, int32_t* status, DeferredRanks dr) {
  static_assert(LDS_INTS >= RouteTables<THREADS, DEFER>::kInts, "tables must fit");
  __shared__ int lds[LDS_INTS];
  const int32_t t = blockIdx.x / nchunks;
  const int32_t chunk = blockIdx.x - t * nchunks;
  PairMeta meta;
  fetch_pair_meta(meta, t, k, ids, idx, nullptr);

  RouteTables<THREADS, DEFER> tables;
  tables.load(send, dr, t, E);
  const int32_t g = chunk * THREADS + threadIdx.x;  // 16-channel group within the row
  const bool active = g < ngroups;
  u32x4 a, b;
  {
    // A lane past the row end loads the row's last group (and takes zeros).
    const u32x4* src = x + (int64_t)t * xs + 2 * (int64_t)min(g, ngroups - 1);
    a = src[0];
    b = src[1];
  }
  keep_order();
  const int* base_lds = tables.store(lds);
  if (!active) a = b = u32x4{0u, 0u, 0u, 0u};
  int64_t slot[KMAX];
  float unused_w[KMAX];
  resolve_routes<KMAX>(meta, lds, base_lds, k, E, cap, slot, unused_w, status,
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
  write_deferred<DEFER>(meta, base_lds, dr, t, k, E, chunk == 0);
}

int kmax_for(int32_t k) { return k <= 2 ? 2 : k <= 4 ? 4 : k <= 8 ? 8 : 16; }

// Launch shapes of the bf16 scatter.
//  - Token rows already in the Infinity Cache (read ahead by the layout's
//    ranking launch): the scatter is bound by its row writes alone, and HBM
//    takes them faster from fewer waves in flight, which write a narrower
//    window of destination rows: 64-thread workgroups holding enough LDS
//    that at most kCachedRowsPerCu share a compute unit.
//  - Rows from HBM: 128-thread workgroups.  Grids of at least
//    kSerialMinItems workgroups (bandwidth bound) stage their tables one load
//    at a time per thread and are capped at kUncachedPerCu workgroups per
//    compute unit; smaller, latency-bound grids stage in one round trip at
//    full occupancy.
template <int THREADS, int LDS_INTS, bool DEFER, Staging ORDER>
hipError_t launch_bf16_shape(const void* x, int64_t x_stride, int32_t bs, int32_t hidden,
                             const int32_t* ids, const int32_t* expand_idx, const int32_t* send,
                             int32_t k, int32_t num_experts, void* expand_x,
                             int64_t expand_x_stride, int64_t capacity_rows, int32_t* status,
                             hipStream_t stream, const DeferredRanks& dr) {
  constexpr int kVpt = MOE_DISPATCH_VPT;
  const int32_t nvec = hidden / 8;  // 16-byte vectors per row
  const int32_t nchunks = (nvec + THREADS * kVpt - 1) / (THREADS * kVpt);
  const int32_t n_items = bs * nchunks;
  const dim3 grid((uint32_t)n_items);
  const u32x4* xv = static_cast<const u32x4*>(x);
  u32x4* ov = static_cast<u32x4*>(expand_x);
  const int64_t xs = x_stride / 8, os = expand_x_stride / 8;
#define MOE_SCATTER(KM)                                                                     \
  launch_kernel(dispatch_bf16_kernel<THREADS, kVpt, KM, LDS_INTS, DEFER, ORDER>, grid,      \
      THREADS, stream, xv, xs, nvec, nchunks, ids, expand_idx, send, k, num_experts, ov, os, \
      capacity_rows, status, dr)
  switch (kmax_for(k)) {
    case 2: MOE_SCATTER(2); break;
    case 4: MOE_SCATTER(4); break;
    case 8: MOE_SCATTER(8); break;
    default: MOE_SCATTER(16); break;
  }
#undef MOE_SCATTER
  return hipGetLastError();
}

// LDS ints per workgroup such that `per_cu` workgroups fit a compute
// unit's 160 KB and one more does not (in 512-byte steps).
constexpr int lds_ints_for(int per_cu) { return (163840 / per_cu) / 512 * 512 / 4; }

#ifndef MOE_FP8_PER_CU
#define MOE_FP8_PER_CU 0   // e4m3 scatter workgroups per compute unit (0: no LDS cap)
#endif
constexpr int kFp8PerCu = MOE_FP8_PER_CU;
#ifndef MOE_FP8_SCATTER_THREADS
#define MOE_FP8_SCATTER_THREADS MOE_FP8_THREADS   // threads per e4m3 scatter workgroup
#endif
constexpr int kFp8Threads = MOE_FP8_SCATTER_THREADS;

template <bool DEFER>
hipError_t launch_fp8_shape(const void* x, int64_t x_stride, int32_t bs, int32_t hidden,
                            const int32_t* ids, const int32_t* expand_idx, const int32_t* send,
                            int32_t k, int32_t num_experts, void* expand_x,
                            int64_t expand_x_stride, int64_t capacity_rows, float* quant_scales,
                            int32_t* status, hipStream_t stream, const DeferredRanks& dr) {
  constexpr int kThreads = kFp8Threads;
  const int32_t ngroups = hidden / 16;
  const int32_t nchunks = (ngroups + kThreads - 1) / kThreads;
  const int32_t n_items = bs * nchunks;
  const dim3 grid((uint32_t)n_items);
  const u32x4* xv = static_cast<const u32x4*>(x);
  u32x4* ov = static_cast<u32x4*>(expand_x);
  const int64_t xs = x_stride / 8, os = expand_x_stride / 16;
  const int32_t nblk = hidden / 128;
  constexpr int kTables = RouteTables<kThreads, DEFER>::kInts;
  constexpr int kLds = kFp8PerCu > 0 && lds_ints_for(kFp8PerCu) > kTables
                           ? lds_ints_for(kFp8PerCu) : kTables;
#define MOE_SCATTER(KM)                                                                     \
  launch_kernel(dispatch_fp8_kernel<kThreads, KM, DEFER, kLds>, grid, kThreads, stream, xv, \
      xs, ngroups, nchunks, ids, expand_idx, send, k, num_experts, ov, os, quant_scales,    \
      nblk, capacity_rows, status, dr)
  switch (kmax_for(k)) {
    case 2: MOE_SCATTER(2); break;
    case 4: MOE_SCATTER(4); break;
    case 8: MOE_SCATTER(8); break;
    default: MOE_SCATTER(16); break;
  }
#undef MOE_SCATTER
  return hipGetLastError();
}


#ifndef MOE_CACHED_ROWS_PER_CU
#define MOE_CACHED_ROWS_PER_CU 7   // workgroups of the cache-resident scatter per compute unit
#endif
constexpr int kCachedRowsThreads = 64;
constexpr int kCachedRowsPerCu = MOE_CACHED_ROWS_PER_CU;
constexpr int kCachedRowsLdsInts = lds_ints_for(kCachedRowsPerCu);
static_assert((kCachedRowsPerCu + 1) * kCachedRowsLdsInts * 4 > 163840, "cap");
#ifndef MOE_UNCACHED_PER_CU
#define MOE_UNCACHED_PER_CU 12     // large HBM-bound grids: workgroups per compute unit
#endif
constexpr int kUncachedPerCu = MOE_UNCACHED_PER_CU;
constexpr int kUncachedLdsInts = lds_ints_for(kUncachedPerCu);

}  // namespace

hipError_t launch_dispatch_bf16(const void* x, int64_t x_stride, int32_t bs, int32_t hidden,
                                const int32_t* ids, const int32_t* expand_idx,
                                const int32_t* send, int32_t k, int32_t num_experts,
                                void* expand_x, int64_t expand_x_stride, int64_t capacity_rows,
                                int32_t* status, hipStream_t stream, bool rows_cached,
                                const DeferredRanks& dr) {
  constexpr int kT = MOE_DISPATCH_THREADS;
  const int64_t items = (int64_t)bs * ((hidden / 8 + kT - 1) / kT);
  const bool big = items >= kSerialMinItems;
#define MOE_SHAPE(TH, LDS, DEF, ORD)                                                      \
  return launch_bf16_shape<TH, LDS, DEF, ORD>(x, x_stride, bs, hidden, ids, expand_idx,   \
      send, k, num_experts, expand_x, expand_x_stride, capacity_rows, status, stream, dr)
  if (rows_cached) {
    if (dr.base) MOE_SHAPE(kCachedRowsThreads, kCachedRowsLdsInts, true, Staging::kTablesFirst);
    MOE_SHAPE(kCachedRowsThreads, kCachedRowsLdsInts, false, Staging::kTablesFirst);
  }
  constexpr int kLdsD = RouteTables<kT, true>::kInts;
  constexpr int kLdsN = RouteTables<kT, false>::kInts;
  constexpr int kCapD = kUncachedLdsInts > kLdsD ? kUncachedLdsInts : kLdsD;
  constexpr int kCapN = kUncachedLdsInts > kLdsN ? kUncachedLdsInts : kLdsN;
  if (big) {
    if (dr.base) MOE_SHAPE(kT, kCapD, true, Staging::kRowsFirstSerial);
    MOE_SHAPE(kT, kCapN, false, Staging::kRowsFirstSerial);
  }
  if (dr.base) MOE_SHAPE(kT, kLdsD, true, Staging::kRowsFirst);
  MOE_SHAPE(kT, kLdsN, false, Staging::kRowsFirst);
#undef MOE_SHAPE
}

hipError_t launch_dispatch_fp8(const void* x, int64_t x_stride, int32_t bs, int32_t hidden,
                               const int32_t* ids, const int32_t* expand_idx,
                               const int32_t* send, int32_t k, int32_t num_experts,
                               void* expand_x, int64_t expand_x_stride, int64_t capacity_rows,
                               float* quant_scales, int32_t* status, hipStream_t stream,
                               const DeferredRanks& dr) {
  if (dr.base)
    return launch_fp8_shape<true>(x, x_stride, bs, hidden, ids, expand_idx, send, k,
                                  num_experts, expand_x, expand_x_stride, capacity_rows,
                                  quant_scales, status, stream, dr);
  return launch_fp8_shape<false>(x, x_stride, bs, hidden, ids, expand_idx, send, k, num_experts,
                                 expand_x, expand_x_stride, capacity_rows, quant_scales, status,
                                 stream, dr);
}

}  // namespace moe
