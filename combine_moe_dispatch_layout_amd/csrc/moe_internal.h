// moe_internal.h -- declarations shared by the library's translation units:
// 16-byte vector type, bf16 helpers, and the kernel launchers that the C ABI
// in api.hip calls after validating its arguments.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_dispatch.h"  // include/ (on the include path)

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
__device__ __forceinline__ float bf16hi_to_f32(uint32_t w) {
  return __uint_as_float(w & 0xFFFF0000u);
}

// fp32 -> bf16 bits, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x0040u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Launch shapes and cache hints of the streaming kernels, chosen by
// measurement on MI355X; each can be overridden at build time.
#ifndef MOE_DISPATCH_THREADS
#define MOE_DISPATCH_THREADS 128   // threads per dispatch workgroup
#endif
#ifndef MOE_DISPATCH_VPT
#define MOE_DISPATCH_VPT 1         // 16-byte vectors per thread per row chunk
#endif
#ifndef MOE_COMBINE_THREADS
#define MOE_COMBINE_THREADS 128
#endif
#ifndef MOE_COMBINE_VPT
#define MOE_COMBINE_VPT 1
#endif
#ifndef MOE_FP8_THREADS
#define MOE_FP8_THREADS 256
#endif
#ifndef MOE_FUSED_THREADS
#define MOE_FUSED_THREADS 256      // threads per one-launch layout + bf16 scatter workgroup
#endif
#ifndef MOE_NT_STORES
#define MOE_NT_STORES 1            // write-once outputs bypass cache retention
#endif
#ifndef MOE_NT_LOADS
#define MOE_NT_LOADS 1             // read-once expert rows bypass cache retention
#endif

template <typename T>
__device__ __forceinline__ void store_stream(T v, T* p) {
#if MOE_NT_STORES
  __builtin_nontemporal_store(v, p);
#else
  *p = v;
#endif
}

template <typename T>
__device__ __forceinline__ T load_stream(const T* p) {
#if MOE_NT_LOADS
  return __builtin_nontemporal_load(p);
#else
  return *p;
#endif
}

// Per-token routing metadata, fetched lane-parallel: lane j < k holds pair
// (t, j)'s expert id, within-expert rank and weight.  Loads are only issued
// here; the values are consumed by resolve_routes.
struct PairMeta {
  int e = -1;
  int r = -1;
  float w = 0.0f;
};

__device__ __forceinline__ void fetch_pair_meta(PairMeta& m, int32_t t, int32_t k,
                                                const int32_t* __restrict__ ids,
                                                const int32_t* __restrict__ idx,
                                                const float* __restrict__ scales) {
  const int lane = threadIdx.x & (kWave - 1);
  if (lane < k) {
    const int64_t p = (int64_t)t * k + lane;
    m.e = ids[p];
    m.r = idx[p];
    if (scales) m.w = scales[p];
  }
}

// Turns fetched metadata into workgroup-uniform routes: destination row
// slot[j] (-1 = pair skipped) and weight w[j], using the send counts staged
// in LDS (plus, when `base_lds` is given, the column prefix of the ranking
// workgroup that ranked the token, for ranks left within that workgroup).
// A slot outside [0, cap) is skipped and, when `report` is set, flagged
// through `status`.
template <int KMAX>
__device__ __forceinline__ void resolve_routes(const PairMeta& m, const int* send_lds,
                                               const int* base_lds, int32_t k, int32_t E,
                                               int64_t cap, int64_t (&slot)[KMAX],
                                               float (&w)[KMAX], int32_t* status, bool report) {
  const int lane = threadIdx.x & (kWave - 1);
  int64_t my_slot = -1;
  if (lane < k && m.e >= 0 && m.e < E && m.r >= 0) {
    const int64_t s = (int64_t)send_lds[m.e] + (base_lds ? base_lds[m.e] : 0) + m.r;
    if (s >= 0 && s < cap)
      my_slot = s;
    else if (report && status)
      atomicOr(status, (int)MOE_FLAG_GUARD);
  }
  const int32_t lo = (int32_t)(my_slot & 0xFFFFFFFF);
  const int32_t hi = (int32_t)(my_slot >> 32);
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    const uint32_t l = (uint32_t)__builtin_amdgcn_readlane(lo, j);
    const int32_t h = __builtin_amdgcn_readlane(hi, j);
    slot[j] = (j < k) ? (int64_t)(((uint64_t)(uint32_t)h << 32) | l) : -1;
    w[j] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m.w), j));
  }
}

// e4m3 quantisation of 16 consecutive bf16 channels held in two 16-byte
// vectors.  The 8 lanes of an aligned lane octet hold one 128-channel block
// and share its scale s = amax / 448 (a correctly rounded division); each
// code is e4m3(x / s), rounded to nearest even by the hardware conversion
// after an exact clamp to +-448.  An all-zero block gives s = 0 and zero
// codes.  Every lane of the wave must take part (the maxima are exchanged
// across lanes); lanes without data pass zeros.
__device__ __forceinline__ u32x4 quantize16_e4m3(const u32x4& a, const u32x4& b, float& s_out) {
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
  s_out = s;
  return codes;
}

// Copies n ints (1 <= n <= N) from global memory into LDS with a
// THREADS-wide workgroup in two steps, so that a caller can put other loads
// between them: load() issues every load into registers, store() writes them
// to LDS (the caller synchronises).  Staging then costs one memory round
// trip.  Neither step branches (a lane past the end repeats element n - 1
// and stores it past the end, into the kSlots-int LDS area), so a wait for
// these loads need not cover loads the caller issues after them.
template <int THREADS, int N>
struct StagedInts {
  static constexpr int kPer = (N + THREADS - 1) / THREADS;
  static constexpr int kSlots = kPer * THREADS;  // LDS ints store() writes
  int v[kPer];
  __device__ __forceinline__ void load(const int32_t* __restrict__ src, int32_t n) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = i * THREADS + (int)threadIdx.x;
      v[i] = src[e < n ? e : n - 1];
    }
  }
  __device__ __forceinline__ void store(int* lds) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) lds[i * THREADS + (int)threadIdx.x] = v[i];
  }
};

// Keeps the compiler from moving memory accesses across this point (no
// instruction is emitted): loads issued before it stay before it, in order.
__device__ __forceinline__ void keep_order() { __asm__ volatile("" ::: "memory"); }

// ep_send_counts[0..E] (E + 1 ints) staged by a THREADS-wide workgroup.
template <int THREADS>
using StagedSend = StagedInts<THREADS, kMaxExperts + 1>;

// Copies ep_send_counts[0..E] into LDS with a workgroup of any size (one
// load per thread and round when blockDim.x >= E + 1).
__device__ __forceinline__ void stage_send_any(int* send_lds, const int32_t* __restrict__ send,
                                               int32_t E) {
  for (int e = threadIdx.x; e <= E; e += blockDim.x) send_lds[e] = send[e];
  __syncthreads();
}

// Zeros read in place of a row that is absent (no shared row), so that the
// load needs no branch.
__device__ const u32x4 kZeroVec = {0u, 0u, 0u, 0u};

// ---- layout ---------------------------------------------------------------
// Ranking workgroups and their work, chosen on the host.
struct LayoutPlan {
  int64_t n_pairs;          // bs * k
  int32_t blocks;           // workgroups of the ranking pass (<= kLayoutMaxBlocks)
  int32_t rounds;           // rounds of kLayoutThreads pairs per chunk
  int32_t chunk_pairs;      // pairs per chunk: whole tokens, at most rounds * kLayoutThreads
  int32_t chunks;           // chunks per ranking workgroup
  int64_t pairs_per_block;  // chunks * chunk_pairs
};
constexpr int kLayoutWaves = 8;
constexpr int kLayoutThreads = kLayoutWaves * kWave;   // 512 pairs per round
#ifndef MOE_LAYOUT_SINGLE_ROUNDS
#define MOE_LAYOUT_SINGLE_ROUNDS 4
#endif
#ifndef MOE_LAYOUT_MULTI_ROUNDS
#define MOE_LAYOUT_MULTI_ROUNDS 4
#endif
// One workgroup ranks up to kLayoutThreads * kLayoutSingleMaxRounds pairs by
// itself; larger batches use workgroups of chunks of kLayoutMultiRounds
// rounds each, at most kLayoutMaxBlocks workgroups (more chunks per
// workgroup beyond that), so the last workgroup's scan over the workgroups'
// histograms stays bounded.
constexpr int kLayoutSingleMaxRounds = MOE_LAYOUT_SINGLE_ROUNDS;
constexpr int kLayoutMultiRounds = MOE_LAYOUT_MULTI_ROUNDS;
constexpr int kLayoutMaxBlocks = 256;

// The multi-workgroup layout's device workspace.  `arrivals` (always the
// workspace's first word) must be zero when a call starts; every call leaves
// it zero again.  The rest needs no initial contents.
struct LayoutScratch {
  int32_t* hist = nullptr;      // [blocks][E] histograms, then their column prefix
  int32_t* flags = nullptr;     // [blocks] status bits per workgroup
  int32_t* arrivals = nullptr;  // workgroups that have published their histogram
  int32_t* ranks = nullptr;     // [n_pairs] ranks within the workgroup (deferred ranks)
};

// Ranks that a multi-workgroup layout left within their ranking workgroup
// (moe_dispatch_fused): the scatter adds the workgroup's column prefix and
// writes the final expand_idx.  base == nullptr: ranks are final.
struct DeferredRanks {
  const int32_t* base = nullptr;  // LayoutScratch::hist after the scan
  int32_t tokens_per_block = 0;   // tokens per ranking workgroup
  int32_t* expand_idx = nullptr;  // final ranks, written by each token's first chunk
};

// Optional logical-expert -> physical-replica choice fused into the ranking
// pass (offsets == nullptr: ids are ranked as given).
struct ReplicaMap {
  const int32_t* offsets = nullptr;      // [n_logical + 1] replica ranges
  const uint32_t* thresholds = nullptr;  // [replicas] cumulative choice thresholds
  int32_t n_logical = 0;
  uint64_t seed = 0;
  int32_t* out = nullptr;                // [n_pairs] chosen replica, -1 if none
};

// Optional per-destination-rank offsets written with the padded scan:
// offsets[r] = send[r * per_rank] for r < ranks, offsets[ranks] = total.
struct RankSplit {
  int32_t* offsets = nullptr;
  int32_t per_rank = 1;
  int32_t ranks = 0;
};

// Token rows that the layout's ranking launch reads ahead.  The layout is
// latency bound and leaves HBM nearly idle, so up to kReadAheadMaxBlocks
// workgroups (together with the ranking workgroups) read the rows the
// scatter will need with ordinary loads, which allocate in the 256 MB
// Infinity Cache; the scatter then finds them there instead of mixing row
// reads from HBM into its write stream.  Token rows of up to
// kReadAheadMaxBytes are read ahead whole; of larger x only the first
// kReadAheadPartBytes, because a partial read-ahead leaves the scatter
// reading the rest from HBM, and a longer one than that was measured slower
// (192 MB of the 235 MB of the 16384-token line: 800 against 794 us per
// step, where reading all 235 MB ahead took 780 us).
struct ReadAhead {
  const u32x4* base = nullptr;
  int64_t vecs = 0;   // 16-byte vectors, from base
};
// Streaming grids of at least this many workgroups (about two full waves of
// workgroups on 256 compute units) are bandwidth bound; smaller ones are
// latency bound.  The scatter of rows from HBM picks its staging by it.
constexpr int64_t kSerialMinItems = 8192;
// Static scratch of moe_dispatch_fused_noalloc, per GPU: enough for the
// layout workspace of any batch of at most 2^20 pairs (E <= 512).
#ifndef MOE_NOALLOC_SCRATCH_BYTES
#define MOE_NOALLOC_SCRATCH_BYTES (size_t(5) << 20)
#endif
#ifndef MOE_READ_AHEAD_BLOCKS
#define MOE_READ_AHEAD_BLOCKS 240  // of the 256 compute units, with the ranking workgroups
#endif
constexpr int kReadAheadMaxBlocks = MOE_READ_AHEAD_BLOCKS;
constexpr int64_t kReadAheadMaxBytes = int64_t(240) << 20;   // of the 256 MB Infinity Cache
constexpr int64_t kReadAheadPartBytes = int64_t(128) << 20;
// Loads in flight per read-ahead thread: enough to keep HBM busy, few enough
// that the ranking workgroups' own loads in the same launch do not queue
// behind a deep backlog.
constexpr int kReadAheadUnroll = 4;

// Body of a read-ahead workgroup: block `blockIdx.x - first_block` of
// `blocks` reads vectors [lo, hi) in spans of blockDim.x * kReadAheadUnroll,
// the workgroups taking neighbouring spans in turn, so that the reads in
// flight form one contiguous front through x rather than one stream per
// workgroup (the front took the layout launch from 14.7 to 13.5 us on the
// 4096-token e4m3 line).  Nothing is stored; the empty asm statement
// consumes the loaded values so the loads are kept.
__device__ __forceinline__ void read_ahead(const ReadAhead& ra, int32_t first_block,
                                           int32_t blocks, int64_t lo, int64_t hi) {
  const int64_t span = (int64_t)blockDim.x * kReadAheadUnroll;
  const int64_t step = (int64_t)blocks * span;
  uint32_t acc = 0;
  for (int64_t v0 = lo + ((int64_t)blockIdx.x - first_block) * span; v0 < hi; v0 += step) {
    u32x4 t[kReadAheadUnroll];
#pragma unroll
    for (int u = 0; u < kReadAheadUnroll; ++u) {
      const int64_t v = v0 + (int64_t)u * blockDim.x + threadIdx.x;
      t[u] = (v < hi) ? ra.base[v] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kReadAheadUnroll; ++u) acc ^= t[u][0] ^ t[u][1] ^ t[u][2] ^ t[u][3];
  }
  __asm__ volatile("" : : "v"(acc));
}

// ---- launches ----------------------------------------------------------------
// Every kernel of the library is launched through launch_kernel.  When the
// calling host thread has event pairs bound by moe_time_next_launches, the
// launch takes the next pair and goes through hipExtLaunchKernel, which
// stamps the two events with the kernel's own start and end; otherwise it is
// a plain launch.
bool take_launch_events(hipEvent_t* start, hipEvent_t* stop);

template <typename... Params, typename... Args>
inline void launch_kernel(void (*kernel)(Params...), dim3 grid, dim3 block, hipStream_t stream,
                          Args... args) {
  static_assert(sizeof...(Params) == sizeof...(Args), "kernel argument count");
  hipEvent_t start = nullptr, stop = nullptr;
  if (take_launch_events(&start, &stop))
    hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, start, stop, 0,
                          static_cast<Params>(args)...);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, stream, static_cast<Params>(args)...);
}

LayoutPlan plan_layout(int32_t bs, int32_t k);

// Read-ahead workgroups only ride along a multi-workgroup layout, and only
// while the ranking workgroups leave compute units free.
inline bool read_ahead_runs(const LayoutPlan& plan, const ReadAhead& ahead) {
  return plan.blocks > 1 && ahead.vecs > 0 && plan.blocks < kReadAheadMaxBlocks;
}
// Contiguous token rows of at least this many bytes (and at most
// kReadAheadMaxBytes) are read ahead before a separate scatter: below it the
// extra launch costs more than the scatter gains from cache-resident rows.
constexpr int64_t kScatterReadAheadMinBytes = int64_t(32) << 20;
// Reads `ahead` into the Infinity Cache in a launch of its own.
hipError_t launch_read_ahead(const ReadAhead& ahead, hipStream_t stream);
size_t layout_workspace_bytes(const LayoutPlan& p, int32_t num_experts);
LayoutScratch layout_scratch(const LayoutPlan& p, int32_t num_experts, void* workspace);

// The layout launch(es).  With defer_ranks and several ranking workgroups,
// only the ranking launch runs: expand_idx is left for a scatter launched
// with the matching DeferredRanks.
hipError_t launch_layout(const int32_t* ids, int32_t k, int32_t num_experts, int32_t align,
                         const LayoutPlan& plan, int32_t* counts, int32_t* send,
                         int32_t* expand_idx, int32_t* status, void* workspace,
                         const ReplicaMap& map, const RankSplit& ranks, hipStream_t stream,
                         const ReadAhead& ahead = ReadAhead{}, bool defer_ranks = false);

// Batches of at most this many pairs fit one layout workgroup; the fused
// layout + bf16 scatter derives the layout in every scatter workgroup.
constexpr int kFusedMaxPairs = kLayoutThreads * kLayoutSingleMaxRounds;

hipError_t launch_dispatch_fused_fp8(const void* x, int64_t x_stride, int32_t bs,
                                     int32_t hidden, const int32_t* ids, int32_t k,
                                     int32_t num_experts, int32_t align, int32_t* counts,
                                     int32_t* send, int32_t* expand_idx, int32_t* status,
                                     void* expand_x, int64_t expand_x_stride,
                                     int64_t capacity_rows, float* quant_scales,
                                     hipStream_t stream);

hipError_t launch_dispatch_fused_bf16(const void* x, int64_t x_stride, int32_t bs,
                                      int32_t hidden, const int32_t* ids, int32_t k,
                                      int32_t num_experts, int32_t align, int32_t* counts,
                                      int32_t* send, int32_t* expand_idx, int32_t* status,
                                      void* expand_x, int64_t expand_x_stride,
                                      int64_t capacity_rows, hipStream_t stream);

// ---- dispatch / combine -----------------------------------------------------
// `expand_idx` holds final ranks, or with deferred.base the ranks within
// the ranking workgroups (then the kernels write deferred.expand_idx).
hipError_t launch_dispatch_bf16(const void* x, int64_t x_stride, int32_t bs, int32_t hidden,
                                const int32_t* ids, const int32_t* expand_idx,
                                const int32_t* send, int32_t k, int32_t num_experts,
                                void* expand_x, int64_t expand_x_stride, int64_t capacity_rows,
                                int32_t* status, hipStream_t stream, bool rows_cached = false,
                                const DeferredRanks& deferred = DeferredRanks{});

hipError_t launch_dispatch_fp8(const void* x, int64_t x_stride, int32_t bs, int32_t hidden,
                               const int32_t* ids, const int32_t* expand_idx,
                               const int32_t* send, int32_t k, int32_t num_experts,
                               void* expand_x, int64_t expand_x_stride, int64_t capacity_rows,
                               float* quant_scales, int32_t* status, hipStream_t stream,
                               const DeferredRanks& deferred = DeferredRanks{});

hipError_t launch_combine(const void* y, int64_t y_stride, int64_t capacity_rows,
                          const int32_t* ids, const int32_t* expand_idx, const int32_t* send,
                          const float* scales, const void* shared, int64_t shared_stride,
                          int32_t bs, int32_t hidden, int32_t k, int32_t num_experts,
                          void* out, int32_t* status, hipStream_t stream);

hipError_t launch_combine_fp8(const void* y, int64_t y_stride, int64_t capacity_rows,
                              const float* y_scales, const int32_t* ids,
                              const int32_t* expand_idx, const int32_t* send,
                              const float* scales, const void* shared, int64_t shared_stride,
                              int32_t bs, int32_t hidden, int32_t k, int32_t num_experts,
                              void* out, int32_t* status, hipStream_t stream);

}  // namespace moe
