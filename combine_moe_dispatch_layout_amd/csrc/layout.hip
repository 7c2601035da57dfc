// layout.hip -- routing -> per-expert counts, 128-padded exclusive prefix sum
// and stable within-expert ranks (the expert_ids / expand_idx /
// ep_send_counts triple of the npu_moe_distribute_combine page; the padding
// is the grouped GEMM's 128-row M-tile from the TEMPO summary, section 1).
//
// Ranking pass (one or more workgroups of 8 waves):
//   The workgroup walks its pairs in rounds of 512 (one per thread) in pair
//   order.  Within a round each wave builds, for every expert it touches, the
//   64-bit mask of its lanes holding that expert (LDS atomic OR: the result
//   does not depend on the order the lanes arrive in).  A lane's rank is then
//     count of that expert in earlier rounds           (run[e])
//   + count in lower-numbered waves of this round      (wcnt[w'][e], w' < w)
//   + popcount(mask & lanes below me).
//   Nothing positional is decided by an atomic race, so the layout is
//   deterministic.  LDS is cleared sparsely: each lowest lane of a group
//   zeroes the one mask / count word it used.
// Single workgroup (<= 8192 pairs): the same kernel also writes the counts and
//   the padded exclusive scan, so small batches take one launch.
// Several workgroups: each writes its expert histogram to the workspace; a
//   second launch gives every workgroup the column sum of the histograms of
//   the workgroups before it (its base per expert), adds that base to its
//   ranks, and the last workgroup (which needs every row anyway) writes the
//   counts, the padded scan and the status word.
#include "moe_internal.h"

namespace moe {
namespace {

// Exclusive scan of one int per thread over a kLayoutThreads workgroup.
__device__ int block_exclusive_scan(int v, int* wave_tot, int* total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  int incl = v;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int o = __shfl_up(incl, d, kWave);
    if (lane >= d) incl += o;
  }
  if (lane == kWave - 1) wave_tot[wave] = incl;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kLayoutWaves; ++w) {
    const int s = wave_tot[w];
    before += (w < wave) ? s : 0;
    all += s;
  }
  __syncthreads();
  *total = all;
  return before + incl - v;
}

// Thread e holds c_e (0 for e >= E).  Writes counts[e], send[e] and send[E].
__device__ void write_counts_and_offsets(int c, int32_t E, int32_t align, int* wave_tot,
                                         int32_t* __restrict__ counts,
                                         int32_t* __restrict__ send) {
  const int e = threadIdx.x;
  const int padded = (c + align - 1) & ~(align - 1);
  int total;
  const int excl = block_exclusive_scan(padded, wave_tot, &total);
  if (e < E) {
    counts[e] = c;
    send[e] = excl;
  }
  if (e == 0) send[E] = total;
}

__global__ __launch_bounds__(kLayoutThreads) void layout_rank_kernel(
    const int32_t* __restrict__ ids, int32_t n_pairs, int32_t k, int32_t E, int32_t align,
    int32_t rounds, int32_t pairs_per_block, int32_t* __restrict__ expand_idx,
    int32_t* __restrict__ block_hist, int32_t* __restrict__ block_flags,
    int32_t* __restrict__ counts, int32_t* __restrict__ send, int32_t* __restrict__ status) {
  __shared__ unsigned long long mask[kLayoutWaves][kMaxExperts];  // 32 KB
  __shared__ int wcnt[kLayoutWaves][kMaxExperts];                 // 16 KB
  __shared__ int run[kMaxExperts];
  __shared__ int wave_tot[kLayoutWaves];
  __shared__ int flags_lds;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int begin = blockIdx.x * pairs_per_block;
  const int end = min(n_pairs, begin + pairs_per_block);

  // Ids are prefetched one round ahead, so a round's global load latency
  // overlaps the previous round's LDS work.
  int e_next = 0;
  {
    const int i0 = begin + tid;
    if (rounds > 0 && i0 < end) e_next = ids[i0];
  }

  for (int j = tid; j < kLayoutWaves * kMaxExperts; j += kLayoutThreads) {
    (&mask[0][0])[j] = 0ull;
    (&wcnt[0][0])[j] = 0;
  }
  for (int j = tid; j < kMaxExperts; j += kLayoutThreads) run[j] = 0;
  if (tid == 0) flags_lds = 0;
  __syncthreads();

  int fl = 0;
  for (int r = 0; r < rounds; ++r) {  // rounds is workgroup-uniform
    const int i = begin + r * kLayoutThreads + tid;
    const bool in = i < end;
    const int e = e_next;
    {
      const int in_next = i + kLayoutThreads;
      e_next = (r + 1 < rounds && in_next < end) ? ids[in_next] : 0;
    }
    const bool ok = in && e >= 0 && e < E;
    if (in && !ok) fl |= MOE_FLAG_ID_RANGE;
    if (ok) {
      for (int j = i - (i % k); j < i; ++j)
        if (ids[j] == e) fl |= MOE_FLAG_DUP_ID;
      atomicOr(&mask[wave][e], 1ull << lane);
    }
    __syncthreads();
    unsigned long long m = 0;
    int lr = 0;
    if (ok) {
      m = mask[wave][e];
      lr = __popcll(m & ((1ull << lane) - 1ull));
      if (lr == 0) wcnt[wave][e] = __popcll(m);
    }
    __syncthreads();
    int rank = -1;
    if (ok) {
      rank = run[e] + lr;
      for (int w = 0; w < wave; ++w) rank += wcnt[w][e];
    }
    __syncthreads();
    if (ok && lr == 0) {
      atomicAdd(&run[e], __popcll(m));
      mask[wave][e] = 0ull;
      wcnt[wave][e] = 0;
    }
    if (in) expand_idx[i] = rank;
  }
  if (fl) atomicOr(&flags_lds, fl);
  __syncthreads();

  if (block_hist == nullptr) {
    // The whole batch was this workgroup: finish the layout here.
    const int c = (tid < E) ? run[tid] : 0;
    write_counts_and_offsets(c, E, align, wave_tot, counts, send);
    if (tid == 0 && status) *status = flags_lds;
  } else {
    for (int e = tid; e < E; e += kLayoutThreads) block_hist[blockIdx.x * E + e] = run[e];
    if (tid == 0) block_flags[blockIdx.x] = flags_lds;
  }
}

__global__ __launch_bounds__(kLayoutThreads) void layout_finalize_kernel(
    const int32_t* __restrict__ ids, int32_t n_pairs, int32_t E, int32_t align,
    int32_t pairs_per_block, int32_t nblocks, const int32_t* __restrict__ block_hist,
    const int32_t* __restrict__ block_flags, int32_t* __restrict__ expand_idx,
    int32_t* __restrict__ counts, int32_t* __restrict__ send, int32_t* __restrict__ status) {
  __shared__ int base[kMaxExperts];
  __shared__ int wave_tot[kLayoutWaves];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const bool last = (b == nblocks - 1);

  int own = 0;
  if (tid < E) {
    int s = 0;
    for (int bb = 0; bb < b; ++bb) s += block_hist[bb * E + tid];
    base[tid] = s;
    if (last) own = s + block_hist[b * E + tid];
  }
  if (last) {  // workgroup-uniform
    write_counts_and_offsets(own, E, align, wave_tot, counts, send);
    if (tid == 0 && status) {
      int f = 0;
      for (int bb = 0; bb < nblocks; ++bb) f |= block_flags[bb];
      *status = f;
    }
  }
  __syncthreads();

  const int begin = b * pairs_per_block;
  const int end = min(n_pairs, begin + pairs_per_block);
  for (int i = begin + tid; i < end; i += kLayoutThreads) {
    const int r = expand_idx[i];
    if (r >= 0) expand_idx[i] = r + base[ids[i]];
  }
}

}  // namespace

LayoutPlan plan_layout(int32_t bs, int32_t k) {
  LayoutPlan p;
  p.n_pairs = (int64_t)bs * k;
  if (p.n_pairs <= (int64_t)kLayoutThreads * kLayoutSingleMaxRounds) {
    p.blocks = 1;
    p.rounds = (int32_t)((p.n_pairs + kLayoutThreads - 1) / kLayoutThreads);
  } else {
    p.rounds = kLayoutMultiRounds;
    const int64_t ppb = (int64_t)kLayoutMultiRounds * kLayoutThreads;
    p.blocks = (int32_t)((p.n_pairs + ppb - 1) / ppb);
  }
  p.pairs_per_block = (int64_t)p.rounds * kLayoutThreads;
  return p;
}

size_t layout_workspace_bytes(const LayoutPlan& p, int32_t num_experts) {
  if (p.blocks <= 1) return 0;
  const size_t hist = (size_t)p.blocks * num_experts * sizeof(int32_t);
  const size_t hist_aligned = (hist + 255) & ~(size_t)255;
  return hist_aligned + (size_t)p.blocks * sizeof(int32_t);
}

hipError_t launch_layout(const int32_t* ids, int32_t k, int32_t num_experts, int32_t align,
                         const LayoutPlan& plan, int32_t* counts, int32_t* send,
                         int32_t* expand_idx, int32_t* status, void* workspace,
                         hipStream_t stream) {
  const int32_t n = (int32_t)plan.n_pairs;
  const int32_t ppb = (int32_t)plan.pairs_per_block;
  if (plan.blocks <= 1) {
    layout_rank_kernel<<<1, kLayoutThreads, 0, stream>>>(ids, n, k, num_experts, align,
                                                         plan.rounds, ppb, expand_idx, nullptr,
                                                         nullptr, counts, send, status);
    return hipGetLastError();
  }
  int32_t* hist = static_cast<int32_t*>(workspace);
  const size_t hist_bytes = ((size_t)plan.blocks * num_experts * sizeof(int32_t) + 255) &
                            ~(size_t)255;
  int32_t* bflags = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + hist_bytes);
  layout_rank_kernel<<<plan.blocks, kLayoutThreads, 0, stream>>>(
      ids, n, k, num_experts, align, plan.rounds, ppb, expand_idx, hist, bflags, counts, send,
      status);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  layout_finalize_kernel<<<plan.blocks, kLayoutThreads, 0, stream>>>(
      ids, n, num_experts, align, ppb, plan.blocks, hist, bflags, expand_idx, counts, send,
      status);
  return hipGetLastError();
}

}  // namespace moe
