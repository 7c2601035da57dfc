// api.hip -- the C ABI declared in include/moe_dispatch.h: host-side argument
// checks, workspace sizing and kernel launches.  No call allocates or
// synchronises, and none keeps state between calls beyond the timing event
// pairs that moe_time_next_launches (include/moe_probe.h) binds per host
// thread.
//
// Argument rules (each failure returns MOE_ERR_INVALID_ARG and enqueues
// nothing): the npu_moe_distribute_combine page gives 1 <= num_experts <= 512,
// 0 < K <= num_experts with K at most 16 (its widest top-K limit), and H a
// positive multiple of 32; the page's per-product caps (BS <= 256/512,
// H <= 7168) are not adopted.  The library adds: bs >= 0, align a power of two
// in [1, 1024], bs*k and the padded capacity at most 2^30 (so 32-bit pair
// indices keep headroom), H <= 65536 (a
// multiple of 128 for e4m3 output), bs*hidden/8 < 2^31, 16-byte aligned row
// bases and strides.
#include <stddef.h>
#include <stdint.h>

#include "moe_internal.h"
#include "moe_probe.h"


namespace {

constexpr int kAbiVersion = 2;

bool is_pow2(int32_t v) { return v > 0 && (v & (v - 1)) == 0; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t capacity_rows_for(int32_t bs, int32_t k, int32_t num_experts, int32_t align) {
  const int64_t n = (int64_t)bs * k;
  const int64_t used = n < num_experts ? n : num_experts;
  return (int64_t)align * ((n + (int64_t)(align - 1) * used) / align);
}

bool layout_args_ok(int32_t bs, int32_t k, int32_t num_experts, int32_t align) {
  if (bs < 0) return false;
  if (num_experts < 1 || num_experts > moe::kMaxExperts) return false;
  if (k < 1 || k > moe::kMaxTopK || k > num_experts) return false;
  if (!is_pow2(align) || align > 1024) return false;
  if (capacity_rows_for(bs, k, num_experts, align) > moe::kMaxRows) return false;
  return true;
}

// Row rules shared by dispatch and combine; elem = bytes per element.
bool row_ok(const void* base, int64_t stride, int32_t hidden, int elem) {
  if (base == nullptr || !aligned16(base)) return false;
  if (stride < hidden || ((stride * elem) & 15) != 0) return false;
  return true;
}

// Work items of the streaming kernels are indexed in 32 bits.
bool rows_fit(int32_t bs, int32_t hidden) { return (int64_t)bs * (hidden / 8) <= INT32_MAX; }

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// Event pairs bound by moe_time_next_launches, per host thread; pairs
// [next, n) are still to be taken by launches.
constexpr int kMaxTimedLaunches = 16;
struct TimedLaunches {
  hipEvent_t start[kMaxTimedLaunches];
  hipEvent_t stop[kMaxTimedLaunches];
  int n = 0;
  int next = 0;
};
thread_local TimedLaunches tl_timed;

// Row and scale rules of the scatter's inputs and outputs (bs > 0).  With no
// capacity nothing is written (every pair is guarded), so the output buffers
// may then be absent.
int scatter_args_check(const void* x, int64_t x_stride, int32_t hidden, const void* expand_x,
                       int64_t expand_x_stride, int64_t capacity_rows, int32_t out_dtype,
                       const float* quant_scales) {
  if (!row_ok(x, x_stride, hidden, 2)) return MOE_ERR_INVALID_ARG;
  if (capacity_rows > 0 &&
      !row_ok(expand_x, expand_x_stride, hidden, out_dtype == MOE_BF16 ? 2 : 1))
    return MOE_ERR_INVALID_ARG;
  if (capacity_rows > 0 && out_dtype == MOE_FP8_E4M3 &&
      (quant_scales == nullptr || (reinterpret_cast<uintptr_t>(quant_scales) & 3u) != 0))
    return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

// The layout over `ranked` experts (through the replica map when it has
// one), then the scatter of x by `route_ids` (the ids the layout ranked:
// expert_ids, or the replica ids it writes), on one stream.  With several
// ranking workgroups this is two launches: the ranking launch, whose last
// workgroup also scans the histograms and whose spare workgroups read
// contiguous token rows ahead (all of them up to kReadAheadMaxBytes, else
// the first kReadAheadPartBytes), and the scatter, which adds each token's
// workgroup prefix to its ranks and writes expand_idx.  When every row was
// read ahead, the bf16 scatter takes its cache-resident launch shape.
int layout_then_scatter(const void* x, int64_t x_stride, int32_t bs, int32_t hidden,
                        const int32_t* expert_ids, const int32_t* route_ids, int32_t k,
                        int32_t ranked, int32_t align, const moe::LayoutPlan& plan,
                        int32_t* counts, int32_t* send, int32_t* expand_idx, void* expand_x,
                        int64_t expand_x_stride, int64_t capacity_rows, int32_t out_dtype,
                        float* quant_scales, int32_t* status, void* workspace,
                        size_t workspace_bytes, const moe::ReplicaMap& map, hipStream_t s) {
  const size_t need = moe::layout_workspace_bytes(plan, ranked);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need || !aligned16(workspace)))
    return MOE_ERR_WORKSPACE;
  moe::ReadAhead ahead;
  bool rows_cached = false;  // every token row read ahead
  if (bs > 0 && x_stride == hidden) {
    const int64_t vecs = (int64_t)bs * hidden / 8;
    ahead.base = static_cast<const moe::u32x4*>(x);
    ahead.vecs = vecs <= moe::kReadAheadMaxBytes / 16 ? vecs : moe::kReadAheadPartBytes / 16;
    rows_cached = ahead.vecs == vecs && moe::read_ahead_runs(plan, ahead);
  }
  // With several ranking workgroups the ranks are left to the scatter (no
  // finalize launch).
  const bool defer = plan.blocks > 1;
  hipError_t err = moe::launch_layout(expert_ids, k, ranked, align, plan, counts, send,
                                      expand_idx, status, workspace, map, moe::RankSplit{}, s,
                                      ahead, defer);
  if (err != hipSuccess || bs == 0) return hip_status(err);
  moe::DeferredRanks dr;
  const int32_t* ranks = expand_idx;
  if (defer) {
    const moe::LayoutScratch ws = moe::layout_scratch(plan, ranked, workspace);
    dr.base = ws.hist;
    dr.tokens_per_block = (int32_t)(plan.pairs_per_block / k);
    dr.expand_idx = expand_idx;
    ranks = ws.ranks;
  }
  if (out_dtype == MOE_BF16)
    return hip_status(moe::launch_dispatch_bf16(x, x_stride, bs, hidden, route_ids, ranks, send,
                                                k, ranked, expand_x, expand_x_stride,
                                                capacity_rows, status, s, rows_cached, dr));
  return hip_status(moe::launch_dispatch_fp8(x, x_stride, bs, hidden, route_ids, ranks, send, k,
                                             ranked, expand_x, expand_x_stride, capacity_rows,
                                             quant_scales, status, s, dr));
}

}  // namespace

namespace moe {

bool take_launch_events(hipEvent_t* start, hipEvent_t* stop) {
  TimedLaunches& t = tl_timed;
  if (t.next >= t.n) return false;
  *start = t.start[t.next];
  *stop = t.stop[t.next];
  ++t.next;
  return true;
}

}  // namespace moe

extern "C" {

int moe_abi_version(void) { return kAbiVersion; }

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument (shape, range, pointer or alignment)";
    case MOE_ERR_WORKSPACE: return "workspace smaller than moe_dispatch_layout_workspace_size";
    case MOE_ERR_UNSUPPORTED: return "unsupported dtype";
    case MOE_ERR_HIP: return "HIP launch failed";
    case MOE_ERR_SCRATCH:
      return "batch needs more than the no-allocation entry point's static scratch";
    default: return "unknown status";
  }
}

int64_t moe_dispatch_capacity(int32_t bs, int32_t k, int32_t num_experts, int32_t align) {
  if (!layout_args_ok(bs, k, num_experts, align)) return -1;
  return capacity_rows_for(bs, k, num_experts, align);
}

size_t moe_dispatch_layout_workspace_size(int32_t bs, int32_t k, int32_t num_experts) {
  if (!layout_args_ok(bs, k, num_experts, 1)) return 0;
  return moe::layout_workspace_bytes(moe::plan_layout(bs, k), num_experts);
}

int moe_dispatch_layout(const int32_t* expert_ids, int32_t bs, int32_t k, int32_t num_experts,
                        int32_t align, int32_t* expert_counts, int32_t* ep_send_counts,
                        int32_t* expand_idx, int32_t* status, void* workspace,
                        size_t workspace_bytes, void* stream) {
  if (!layout_args_ok(bs, k, num_experts, align)) return MOE_ERR_INVALID_ARG;
  if (expert_counts == nullptr || ep_send_counts == nullptr) return MOE_ERR_INVALID_ARG;
  if (bs > 0 && (expert_ids == nullptr || expand_idx == nullptr)) return MOE_ERR_INVALID_ARG;
  const moe::LayoutPlan plan = moe::plan_layout(bs, k);
  const size_t need = moe::layout_workspace_bytes(plan, num_experts);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need || !aligned16(workspace)))
    return MOE_ERR_WORKSPACE;
  return hip_status(moe::launch_layout(expert_ids, k, num_experts, align, plan, expert_counts,
                                       ep_send_counts, expand_idx, status, workspace,
                                       moe::ReplicaMap{}, moe::RankSplit{},
                                       static_cast<hipStream_t>(stream)));
}

int moe_dispatch_layout_ep(const int32_t* expert_ids, int32_t bs, int32_t k, int32_t num_experts,
                           int32_t ep_world_size, int32_t align, int32_t* expert_counts,
                           int32_t* ep_send_counts, int32_t* rank_offsets, int32_t* expand_idx,
                           int32_t* status, void* workspace, size_t workspace_bytes,
                           void* stream) {
  if (!layout_args_ok(bs, k, num_experts, align)) return MOE_ERR_INVALID_ARG;
  if (ep_world_size < 1 || ep_world_size > num_experts || num_experts % ep_world_size != 0)
    return MOE_ERR_INVALID_ARG;
  if (expert_counts == nullptr || ep_send_counts == nullptr || rank_offsets == nullptr)
    return MOE_ERR_INVALID_ARG;
  if (bs > 0 && (expert_ids == nullptr || expand_idx == nullptr)) return MOE_ERR_INVALID_ARG;
  const moe::LayoutPlan plan = moe::plan_layout(bs, k);
  const size_t need = moe::layout_workspace_bytes(plan, num_experts);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need || !aligned16(workspace)))
    return MOE_ERR_WORKSPACE;
  moe::RankSplit ranks;
  ranks.offsets = rank_offsets;
  ranks.per_rank = num_experts / ep_world_size;
  ranks.ranks = ep_world_size;
  return hip_status(moe::launch_layout(expert_ids, k, num_experts, align, plan, expert_counts,
                                       ep_send_counts, expand_idx, status, workspace,
                                       moe::ReplicaMap{}, ranks,
                                       static_cast<hipStream_t>(stream)));
}

int moe_dispatch_layout_replicated(const int32_t* expert_ids, int32_t bs, int32_t k,
                                   int32_t num_experts, const int32_t* replica_offsets,
                                   const uint32_t* replica_thresholds, int32_t num_replicas,
                                   uint64_t seed, int32_t align, int32_t* replica_ids,
                                   int32_t* replica_counts, int32_t* ep_send_counts,
                                   int32_t* expand_idx, int32_t* status, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  if (!layout_args_ok(bs, k, num_experts, align)) return MOE_ERR_INVALID_ARG;
  if (!layout_args_ok(bs, k, num_replicas, align)) return MOE_ERR_INVALID_ARG;
  if (replica_counts == nullptr || ep_send_counts == nullptr || replica_offsets == nullptr ||
      replica_thresholds == nullptr)
    return MOE_ERR_INVALID_ARG;
  if (bs > 0 && (expert_ids == nullptr || expand_idx == nullptr || replica_ids == nullptr))
    return MOE_ERR_INVALID_ARG;
  const moe::LayoutPlan plan = moe::plan_layout(bs, k);
  const size_t need = moe::layout_workspace_bytes(plan, num_replicas);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need || !aligned16(workspace)))
    return MOE_ERR_WORKSPACE;
  moe::ReplicaMap map;
  map.offsets = replica_offsets;
  map.thresholds = replica_thresholds;
  map.n_logical = num_experts;
  map.seed = seed;
  map.out = replica_ids;
  return hip_status(moe::launch_layout(expert_ids, k, num_replicas, align, plan, replica_counts,
                                       ep_send_counts, expand_idx, status, workspace, map,
                                       moe::RankSplit{}, static_cast<hipStream_t>(stream)));
}

int moe_dispatch(const void* x, int64_t x_stride, int32_t bs, int32_t hidden,
                 const int32_t* expert_ids, const int32_t* expand_idx,
                 const int32_t* ep_send_counts, int32_t k, int32_t num_experts, void* expand_x,
                 int64_t expand_x_stride, int64_t capacity_rows, int32_t out_dtype,
                 float* quant_scales, int32_t* status, void* stream) {
  if (out_dtype != MOE_BF16 && out_dtype != MOE_FP8_E4M3) return MOE_ERR_UNSUPPORTED;
  if (!layout_args_ok(bs, k, num_experts, 1)) return MOE_ERR_INVALID_ARG;
  if (hidden <= 0 || hidden % 32 != 0 || hidden > 65536) return MOE_ERR_INVALID_ARG;
  if (out_dtype == MOE_FP8_E4M3 && hidden % 128 != 0) return MOE_ERR_INVALID_ARG;
  if (capacity_rows < 0 || !rows_fit(bs, hidden)) return MOE_ERR_INVALID_ARG;
  if (bs == 0) return MOE_OK;
  if (expert_ids == nullptr || expand_idx == nullptr || ep_send_counts == nullptr)
    return MOE_ERR_INVALID_ARG;
  const int err = scatter_args_check(x, x_stride, hidden, expand_x, expand_x_stride,
                                     capacity_rows, out_dtype, quant_scales);
  if (err != MOE_OK) return err;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // Contiguous rows of a bandwidth-bound bf16 batch are read ahead first, so
  // that the scatter writes from cache-resident rows instead of interleaving
  // row reads from HBM with its writes.  (The e4m3 scatter writes half the
  // bytes per row; there the extra launch gains nothing measurable.)
  const int64_t x_bytes = (int64_t)bs * hidden * 2;
  const bool rows_cached = out_dtype == MOE_BF16 && capacity_rows > 0 && x_stride == hidden &&
                           x_bytes >= moe::kScatterReadAheadMinBytes &&
                           x_bytes <= moe::kReadAheadMaxBytes;
  if (rows_cached) {
    moe::ReadAhead ahead;
    ahead.base = static_cast<const moe::u32x4*>(x);
    ahead.vecs = x_bytes / 16;
    const hipError_t err = moe::launch_read_ahead(ahead, s);
    if (err != hipSuccess) return hip_status(err);
  }
  if (out_dtype == MOE_BF16)
    return hip_status(moe::launch_dispatch_bf16(x, x_stride, bs, hidden, expert_ids, expand_idx,
                                                ep_send_counts, k, num_experts, expand_x,
                                                expand_x_stride, capacity_rows, status, s,
                                                rows_cached));
  return hip_status(moe::launch_dispatch_fp8(x, x_stride, bs, hidden, expert_ids, expand_idx,
                                             ep_send_counts, k, num_experts, expand_x,
                                             expand_x_stride, capacity_rows, quant_scales,
                                             status, s));
}

int moe_dispatch_fused(const void* x, int64_t x_stride, int32_t bs, int32_t hidden,
                       const int32_t* expert_ids, int32_t k, int32_t num_experts, int32_t align,
                       int32_t* expert_counts, int32_t* ep_send_counts, int32_t* expand_idx,
                       void* expand_x, int64_t expand_x_stride, int64_t capacity_rows,
                       int32_t out_dtype, float* quant_scales, int32_t* status, void* workspace,
                       size_t workspace_bytes, void* stream) {
  if (out_dtype != MOE_BF16 && out_dtype != MOE_FP8_E4M3) return MOE_ERR_UNSUPPORTED;
  if (!layout_args_ok(bs, k, num_experts, align)) return MOE_ERR_INVALID_ARG;
  if (hidden <= 0 || hidden % 32 != 0 || hidden > 65536) return MOE_ERR_INVALID_ARG;
  if (out_dtype == MOE_FP8_E4M3 && hidden % 128 != 0) return MOE_ERR_INVALID_ARG;
  if (capacity_rows < 0 || !rows_fit(bs, hidden)) return MOE_ERR_INVALID_ARG;
  if (expert_counts == nullptr || ep_send_counts == nullptr) return MOE_ERR_INVALID_ARG;
  if (bs > 0) {
    if (expert_ids == nullptr || expand_idx == nullptr) return MOE_ERR_INVALID_ARG;
    const int err = scatter_args_check(x, x_stride, hidden, expand_x, expand_x_stride,
                                       capacity_rows, out_dtype, quant_scales);
    if (err != MOE_OK) return err;
  }
  const moe::LayoutPlan plan = moe::plan_layout(bs, k);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (bs > 0 && plan.n_pairs <= moe::kFusedMaxPairs) {
    if (out_dtype == MOE_BF16)
      return hip_status(moe::launch_dispatch_fused_bf16(
          x, x_stride, bs, hidden, expert_ids, k, num_experts, align, expert_counts,
          ep_send_counts, expand_idx, status, expand_x, expand_x_stride, capacity_rows, s));
    return hip_status(moe::launch_dispatch_fused_fp8(
        x, x_stride, bs, hidden, expert_ids, k, num_experts, align, expert_counts,
        ep_send_counts, expand_idx, status, expand_x, expand_x_stride, capacity_rows,
        quant_scales, s));
  }
  // Otherwise: the layout launch(es), then the scatter, on the same stream.
  return layout_then_scatter(x, x_stride, bs, hidden, expert_ids, expert_ids, k, num_experts,
                             align, plan, expert_counts, ep_send_counts, expand_idx, expand_x,
                             expand_x_stride, capacity_rows, out_dtype, quant_scales, status,
                             workspace, workspace_bytes, moe::ReplicaMap{}, s);
}

int moe_dispatch_fused_replicated(const void* x, int64_t x_stride, int32_t bs, int32_t hidden,
                                  const int32_t* expert_ids, int32_t k, int32_t num_experts,
                                  const int32_t* replica_offsets,
                                  const uint32_t* replica_thresholds, int32_t num_replicas,
                                  uint64_t seed, int32_t align, int32_t* replica_ids,
                                  int32_t* replica_counts, int32_t* ep_send_counts,
                                  int32_t* expand_idx, void* expand_x, int64_t expand_x_stride,
                                  int64_t capacity_rows, int32_t out_dtype, float* quant_scales,
                                  int32_t* status, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  if (out_dtype != MOE_BF16 && out_dtype != MOE_FP8_E4M3) return MOE_ERR_UNSUPPORTED;
  if (!layout_args_ok(bs, k, num_experts, align)) return MOE_ERR_INVALID_ARG;
  if (!layout_args_ok(bs, k, num_replicas, align)) return MOE_ERR_INVALID_ARG;
  if (hidden <= 0 || hidden % 32 != 0 || hidden > 65536) return MOE_ERR_INVALID_ARG;
  if (out_dtype == MOE_FP8_E4M3 && hidden % 128 != 0) return MOE_ERR_INVALID_ARG;
  if (capacity_rows < 0 || !rows_fit(bs, hidden)) return MOE_ERR_INVALID_ARG;
  if (replica_counts == nullptr || ep_send_counts == nullptr || replica_offsets == nullptr ||
      replica_thresholds == nullptr)
    return MOE_ERR_INVALID_ARG;
  if (bs > 0) {
    if (expert_ids == nullptr || expand_idx == nullptr || replica_ids == nullptr)
      return MOE_ERR_INVALID_ARG;
    const int err = scatter_args_check(x, x_stride, hidden, expand_x, expand_x_stride,
                                       capacity_rows, out_dtype, quant_scales);
    if (err != MOE_OK) return err;
  }
  const moe::LayoutPlan plan = moe::plan_layout(bs, k);
  moe::ReplicaMap map;
  map.offsets = replica_offsets;
  map.thresholds = replica_thresholds;
  map.n_logical = num_experts;
  map.seed = seed;
  map.out = replica_ids;
  return layout_then_scatter(x, x_stride, bs, hidden, expert_ids, replica_ids, k, num_replicas,
                             align, plan, replica_counts, ep_send_counts, expand_idx, expand_x,
                             expand_x_stride, capacity_rows, out_dtype, quant_scales, status,
                             workspace, workspace_bytes, map, static_cast<hipStream_t>(stream));
}

int moe_combine(const void* expand_x, int64_t expand_x_stride, int64_t capacity_rows,
                const int32_t* expert_ids, const int32_t* expand_idx,
                const int32_t* ep_send_counts, const float* expert_scales,
                const void* shared_expert_x, int64_t shared_stride, int32_t bs, int32_t hidden,
                int32_t k, int32_t num_experts, void* x_out, int32_t* status, void* stream) {
  if (!layout_args_ok(bs, k, num_experts, 1)) return MOE_ERR_INVALID_ARG;
  if (hidden <= 0 || hidden % 32 != 0 || hidden > 65536) return MOE_ERR_INVALID_ARG;
  if (capacity_rows < 0 || !rows_fit(bs, hidden)) return MOE_ERR_INVALID_ARG;
  if (bs == 0) return MOE_OK;
  if (expert_ids == nullptr || expand_idx == nullptr || ep_send_counts == nullptr ||
      expert_scales == nullptr)
    return MOE_ERR_INVALID_ARG;
  if (capacity_rows > 0 && !row_ok(expand_x, expand_x_stride, hidden, 2))
    return MOE_ERR_INVALID_ARG;
  if (shared_expert_x != nullptr && !row_ok(shared_expert_x, shared_stride, hidden, 2))
    return MOE_ERR_INVALID_ARG;
  if (!row_ok(x_out, hidden, hidden, 2)) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_combine(expand_x, expand_x_stride, capacity_rows, expert_ids,
                                        expand_idx, ep_send_counts, expert_scales,
                                        shared_expert_x, shared_stride, bs, hidden, k,
                                        num_experts, x_out, status,
                                        static_cast<hipStream_t>(stream)));
}

int moe_combine_fp8(const void* expand_x, int64_t expand_x_stride, int64_t capacity_rows,
                    const float* quant_scales, const int32_t* expert_ids,
                    const int32_t* expand_idx, const int32_t* ep_send_counts,
                    const float* expert_scales, const void* shared_expert_x,
                    int64_t shared_stride, int32_t bs, int32_t hidden, int32_t k,
                    int32_t num_experts, void* x_out, int32_t* status, void* stream) {
  if (!layout_args_ok(bs, k, num_experts, 1)) return MOE_ERR_INVALID_ARG;
  if (hidden <= 0 || hidden % 128 != 0 || hidden > 65536) return MOE_ERR_INVALID_ARG;
  if (capacity_rows < 0 || !rows_fit(bs, hidden)) return MOE_ERR_INVALID_ARG;
  if (bs == 0) return MOE_OK;
  if (expert_ids == nullptr || expand_idx == nullptr || ep_send_counts == nullptr ||
      expert_scales == nullptr)
    return MOE_ERR_INVALID_ARG;
  if (capacity_rows > 0) {
    if (!row_ok(expand_x, expand_x_stride, hidden, 1)) return MOE_ERR_INVALID_ARG;
    if (quant_scales == nullptr || (reinterpret_cast<uintptr_t>(quant_scales) & 3u) != 0)
      return MOE_ERR_INVALID_ARG;
  }
  if (shared_expert_x != nullptr && !row_ok(shared_expert_x, shared_stride, hidden, 2))
    return MOE_ERR_INVALID_ARG;
  if (!row_ok(x_out, hidden, hidden, 2)) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_combine_fp8(expand_x, expand_x_stride, capacity_rows,
                                            quant_scales, expert_ids, expand_idx,
                                            ep_send_counts, expert_scales, shared_expert_x,
                                            shared_stride, bs, hidden, k, num_experts, x_out,
                                            status, static_cast<hipStream_t>(stream)));
}

int moe_time_next_launches(void* const* start_events, void* const* stop_events, int32_t n) {
  if (n < 0 || n > kMaxTimedLaunches) return MOE_ERR_INVALID_ARG;
  if (n > 0 && (start_events == nullptr || stop_events == nullptr)) return MOE_ERR_INVALID_ARG;
  for (int32_t i = 0; i < n; ++i)
    if (start_events[i] == nullptr || stop_events[i] == nullptr) return MOE_ERR_INVALID_ARG;
  TimedLaunches& t = tl_timed;
  for (int32_t i = 0; i < n; ++i) {
    t.start[i] = static_cast<hipEvent_t>(start_events[i]);
    t.stop[i] = static_cast<hipEvent_t>(stop_events[i]);
  }
  t.n = n;
  t.next = 0;
  return MOE_OK;
}

int32_t moe_time_unused_launches(void) { return tl_timed.n - tl_timed.next; }

}  // extern "C"
