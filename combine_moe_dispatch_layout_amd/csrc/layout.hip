// layout.hip -- routing -> per-expert counts, 128-padded exclusive prefix sum
// and stable within-expert ranks (the expert_ids / expand_idx /
// ep_send_counts triple of the npu_moe_distribute_combine page; the padding
// is the grouped GEMM's 128-row M-tile from the TEMPO summary, section 1).
//
// Ranking pass (one or more workgroups of 8 waves):
//   Wave w of a workgroup owns a contiguous run of 64*R pairs and walks it in
//   R sub-rounds of 64 (one pair per lane), entirely against its own LDS
//   slice, so no workgroup barrier is needed inside the walk:
//     - every lane ORs its bit into mask[w][e] for its expert e (LDS atomic
//       OR: the result does not depend on the order the lanes arrive in);
//     - a lane's local rank = wave_run[w][e] (pairs of e in this wave's
//       earlier sub-rounds) + popcount(mask & lanes below it);
//     - the lowest lane of each expert group advances wave_run[w][e] and
//       clears the mask word.
//   LDS instructions of one wave execute in issue order, so each step sees
//   the previous one.  After one workgroup barrier a per-expert exclusive
//   prefix over the 8 waves turns local ranks into workgroup ranks.  Nothing
//   positional is decided by an atomic race, so the layout is deterministic.
// Repeated ids: each thread checks one token's K ids against each other in
//   registers.
// Single workgroup (<= 2048 pairs): the same kernel also writes the counts and
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

// Thread e holds c_e (0 for e >= E).  Writes counts[e], send[e] and send[E];
// with a rank split also the per-destination-rank offsets send[r * per_rank].
__device__ void write_counts_and_offsets(int c, int32_t E, int32_t align, int* wave_tot,
                                         int32_t* __restrict__ counts,
                                         int32_t* __restrict__ send, const RankSplit& ranks) {
  const int e = threadIdx.x;
  const int padded = (c + align - 1) & ~(align - 1);
  int total;
  const int excl = block_exclusive_scan(padded, wave_tot, &total);
  if (e < E) {
    counts[e] = c;
    send[e] = excl;
    if (ranks.offsets != nullptr && e % ranks.per_rank == 0)
      ranks.offsets[e / ranks.per_rank] = excl;
  }
  if (e == 0) {
    send[E] = total;
    if (ranks.offsets != nullptr) ranks.offsets[ranks.ranks] = total;
  }
}

// Flags an expert (an id in [0, E)) repeated within one of the tokens whose
// first pair lies in [begin, end).
__device__ __forceinline__ int duplicate_flags(const int32_t* __restrict__ ids, int32_t k,
                                               int32_t E, int begin, int end) {
  int fl = 0;
  for (int t = (begin + k - 1) / k + (int)threadIdx.x; t * k < end; t += kLayoutThreads) {
    int v[kMaxTopK];
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) v[j] = (j < k) ? ids[t * k + j] : -1 - j;
#pragma unroll
    for (int a = 1; a < kMaxTopK; ++a)
#pragma unroll
      for (int b = 0; b < a; ++b)
        if (a < k && v[a] == v[b] && v[a] >= 0 && v[a] < E) fl = MOE_FLAG_DUP_ID;
  }
  return fl;
}

// SplitMix64 draw i of the stream seeded with `seed` (Steele, Lea and Flood,
// OOPSLA 2014): the state seed + (i+1)*golden-gamma through the variant-13
// finaliser.  Counter-based, so every pair computes its own draw.
__device__ __forceinline__ uint64_t splitmix64(uint64_t seed, uint64_t i) {
  uint64_t z = seed + (i + 1u) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Ranking over E "experts".  With a replica map, ids are logical experts in
// [0, map.n_logical) and each pair is first sent to one of its expert's
// physical replicas (E = number of replicas): u = upper 32 bits of the pair's
// SplitMix64 draw, replica = first r of the expert's range with
// u <= thresholds[r] (TEMPO summary, section 2: probabilistic replica
// dispatch and count gathering in one in-graph kernel).
template <int R>
__global__ __launch_bounds__(kLayoutThreads) void layout_rank_kernel(
    const int32_t* __restrict__ ids, int32_t n_pairs, int32_t k, int32_t E, int32_t align,
    int32_t* __restrict__ expand_idx, int32_t* __restrict__ block_hist,
    int32_t* __restrict__ block_flags, int32_t* __restrict__ counts, int32_t* __restrict__ send,
    int32_t* __restrict__ status, ReplicaMap map, RankSplit ranks, ReadAhead ahead,
    int32_t rank_blocks, int32_t ahead_blocks) {
  if ((int32_t)blockIdx.x >= rank_blocks) {  // read-ahead workgroup: vectors [0, split)
    read_ahead(ahead, rank_blocks, ahead_blocks, 0, ahead.split);
    return;
  }
  __shared__ unsigned long long mask[kLayoutWaves][kMaxExperts];  // 32 KB
  __shared__ int wave_run[kLayoutWaves][kMaxExperts];             // 16 KB
  __shared__ int rep_off[kMaxExperts + 1];
  __shared__ uint32_t rep_thr[kMaxExperts];
  __shared__ int wave_tot[kLayoutWaves];
  __shared__ int flags_lds;
  const bool mapped = map.offsets != nullptr;
  const int32_t n_ids = mapped ? map.n_logical : E;  // valid range of the input ids

  constexpr int kPairs = kLayoutThreads * R;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int begin = blockIdx.x * kPairs;
  const int end = min(n_pairs, begin + kPairs);
  const int wbase = begin + wave * (kWave * R);

  // All id loads of this thread first.
  int e[R];
#pragma unroll
  for (int s = 0; s < R; ++s) {
    const int i = wbase + s * kWave + lane;
    e[s] = (i < end) ? ids[i] : 0;
  }

  for (int j = tid; j < kLayoutWaves * kMaxExperts; j += kLayoutThreads) {
    (&mask[0][0])[j] = 0ull;
    (&wave_run[0][0])[j] = 0;
  }
  if (tid == 0) flags_lds = 0;
  if (mapped) {
    for (int j = tid; j <= n_ids; j += kLayoutThreads) rep_off[j] = map.offsets[j];
    for (int j = tid; j < E; j += kLayoutThreads) rep_thr[j] = map.thresholds[j];
  }
  int fl = duplicate_flags(ids, k, n_ids, begin, end);
  __syncthreads();

  if (mapped) {
#pragma unroll
    for (int s = 0; s < R; ++s) {
      const int i = wbase + s * kWave + lane;
      if (i >= end) continue;
      int r = -1;
      if (e[s] >= 0 && e[s] < n_ids) {
        const uint32_t u = (uint32_t)(splitmix64(map.seed, (uint64_t)i) >> 32);
        const int lo = rep_off[e[s]], hi = rep_off[e[s] + 1];
        for (int c = lo; c < hi; ++c)
          if (c >= 0 && c < E && u <= rep_thr[c]) {
            r = c;
            break;
          }
        if (r < 0) fl |= MOE_FLAG_REPLICA;
      } else {
        fl |= MOE_FLAG_ID_RANGE;
      }
      map.out[i] = r;
      e[s] = r;  // ranked as a physical replica; -1 drops the pair
    }
  }

  const unsigned long long below_me = (1ull << lane) - 1ull;
  int lr[R];
#pragma unroll
  for (int s = 0; s < R; ++s) {
    const int i = wbase + s * kWave + lane;
    const bool in = i < end;
    const bool ok = in && e[s] >= 0 && e[s] < E;
    if (in && !ok && !mapped) fl |= MOE_FLAG_ID_RANGE;
    if (ok) atomicOr(&mask[wave][e[s]], 1ull << lane);
    __builtin_amdgcn_wave_barrier();
    unsigned long long m = 0;
    int before = 0;
    if (ok) {
      m = mask[wave][e[s]];
      before = wave_run[wave][e[s]];
    }
    __builtin_amdgcn_wave_barrier();
    const int below = __popcll(m & below_me);
    lr[s] = ok ? before + below : -1;
    if (ok && below == 0) {
      wave_run[wave][e[s]] = before + __popcll(m);
      mask[wave][e[s]] = 0ull;
    }
    __builtin_amdgcn_wave_barrier();
  }
  __syncthreads();

  // Exclusive prefix over waves, per expert; tot = this workgroup's count.
  int tot = 0;
  if (tid < E) {
#pragma unroll
    for (int w = 0; w < kLayoutWaves; ++w) {
      const int c = wave_run[w][tid];
      wave_run[w][tid] = tot;
      tot += c;
    }
  }
  if (fl) atomicOr(&flags_lds, fl);
  __syncthreads();

#pragma unroll
  for (int s = 0; s < R; ++s) {
    const int i = wbase + s * kWave + lane;
    if (i < end) expand_idx[i] = lr[s] >= 0 ? lr[s] + wave_run[wave][e[s]] : -1;
  }

  if (block_hist == nullptr) {
    // The whole batch was this workgroup: finish the layout here.
    write_counts_and_offsets(tot, E, align, wave_tot, counts, send, ranks);
    if (tid == 0 && status) *status = flags_lds;
  } else {
    if (tid < E) block_hist[blockIdx.x * E + tid] = tot;
    if (tid == 0) block_flags[blockIdx.x] = flags_lds;
  }
}

__global__ __launch_bounds__(kLayoutThreads) void layout_finalize_kernel(
    const int32_t* __restrict__ ids, int32_t n_pairs, int32_t E, int32_t align,
    int32_t pairs_per_block, int32_t nblocks, const int32_t* __restrict__ block_hist,
    const int32_t* __restrict__ block_flags, int32_t* __restrict__ expand_idx,
    int32_t* __restrict__ counts, int32_t* __restrict__ send, int32_t* __restrict__ status,
    RankSplit ranks, ReadAhead ahead, int32_t ahead_blocks) {
  if ((int32_t)blockIdx.x >= nblocks) {  // read-ahead workgroup: vectors [split, vecs)
    read_ahead(ahead, nblocks, ahead_blocks, ahead.split, ahead.vecs);
    return;
  }
  __shared__ int base[kMaxExperts];
  __shared__ int wave_tot[kLayoutWaves];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const bool last = (b == nblocks - 1);

  __shared__ int flags_lds;
  if (tid == 0) flags_lds = 0;
  // This workgroup's pairs (the same split as the ranking pass): their loads
  // do not depend on the histograms, so they are issued first and are in
  // flight while the column sums below are formed.
  const int begin = b * pairs_per_block;
  const int end = min(n_pairs, begin + pairs_per_block);
  int r[kLayoutMultiRounds], e[kLayoutMultiRounds];
#pragma unroll
  for (int s = 0; s < kLayoutMultiRounds; ++s) {
    const int i = begin + s * kLayoutThreads + tid;
    r[s] = (i < end) ? expand_idx[i] : -1;
    e[s] = (i < end) ? ids[i] : 0;
  }
  const int mine = (last && tid < E) ? block_hist[b * E + tid] : 0;
  // Column sums over the earlier workgroups' histograms.  When E leaves
  // threads over, `groups` threads share a column (E rounded up to a power
  // of two, at most 16 per column), each summing every groups-th row, so one
  // thread's chain of load batches is groups times shorter; the partial
  // sums meet in LDS.
  __shared__ int part[kLayoutThreads];
  int epad = 1;
  while (epad < E) epad <<= 1;
  const int groups = min(16, kLayoutThreads / epad);  // workgroup-uniform
  int own = 0;
  if (groups == 1) {  // one thread per column: sum directly
    if (tid < E) {
      int sum = 0;
#pragma unroll 8
      for (int bb = 0; bb < b; ++bb) sum += block_hist[bb * E + tid];
      base[tid] = sum;
      own = sum + mine;
    }
  } else {
    const int col = tid & (epad - 1);
    const int grp = tid / epad;
    int sum = 0;
    if (col < E && grp < groups) {
#pragma unroll 8
      for (int bb = grp; bb < b; bb += groups) sum += block_hist[bb * E + col];
    }
    part[tid] = sum;
    __syncthreads();
    if (tid < E) {
      int total = 0;
      for (int g = 0; g < groups; ++g) total += part[g * epad + tid];
      base[tid] = total;
      own = total + mine;
    }
  }
  if (last) {  // workgroup-uniform
    write_counts_and_offsets(own, E, align, wave_tot, counts, send, ranks);
    int f = 0;
    for (int bb = tid; bb < nblocks; bb += kLayoutThreads) f |= block_flags[bb];
    if (f) atomicOr(&flags_lds, f);
    __syncthreads();
    if (tid == 0 && status) *status = flags_lds;
  }
  __syncthreads();

#pragma unroll
  for (int s = 0; s < kLayoutMultiRounds; ++s) {
    const int i = begin + s * kLayoutThreads + tid;
    if (r[s] >= 0) expand_idx[i] = r[s] + base[e[s]];
  }
}

}  // namespace

LayoutPlan plan_layout(int32_t bs, int32_t k) {
  LayoutPlan p;
  p.n_pairs = (int64_t)bs * k;
  if (p.n_pairs <= (int64_t)kLayoutThreads * kLayoutSingleMaxRounds) {
    p.blocks = 1;
    int r = 1;
    while ((int64_t)r * kLayoutThreads < p.n_pairs) r *= 2;
    p.rounds = r;
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

namespace {

template <int R>
void launch_rank(const LayoutPlan& plan, const int32_t* ids, int32_t k, int32_t E, int32_t align,
                 int32_t* expand_idx, int32_t* hist, int32_t* bflags, int32_t* counts,
                 int32_t* send, int32_t* status, const ReplicaMap& map, const RankSplit& ranks,
                 hipStream_t stream, const ReadAhead& ahead, int32_t ahead_blocks) {
  launch_kernel(layout_rank_kernel<R>, plan.blocks + ahead_blocks, kLayoutThreads, stream,
      ids, (int32_t)plan.n_pairs, k, E, align, expand_idx, hist, bflags, counts, send, status,
      map, ranks, ahead, plan.blocks, ahead_blocks);
}

}  // namespace

hipError_t launch_layout(const int32_t* ids, int32_t k, int32_t num_experts, int32_t align,
                         const LayoutPlan& plan, int32_t* counts, int32_t* send,
                         int32_t* expand_idx, int32_t* status, void* workspace,
                         const ReplicaMap& map, const RankSplit& ranks, hipStream_t stream,
                         const ReadAhead& ahead) {
  const int32_t ahead_blocks =
      read_ahead_runs(plan, ahead) ? kReadAheadMaxBlocks - plan.blocks : 0;
  int32_t* hist = nullptr;
  int32_t* bflags = nullptr;
  if (plan.blocks > 1) {
    hist = static_cast<int32_t*>(workspace);
    const size_t hist_bytes = ((size_t)plan.blocks * num_experts * sizeof(int32_t) + 255) &
                              ~(size_t)255;
    bflags = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + hist_bytes);
  }
  switch (plan.rounds) {
    case 1: launch_rank<1>(plan, ids, k, num_experts, align, expand_idx, hist, bflags, counts,
                           send, status, map, ranks, stream, ahead, ahead_blocks); break;
    case 2: launch_rank<2>(plan, ids, k, num_experts, align, expand_idx, hist, bflags, counts,
                           send, status, map, ranks, stream, ahead, ahead_blocks); break;
    case 4: launch_rank<4>(plan, ids, k, num_experts, align, expand_idx, hist, bflags, counts,
                           send, status, map, ranks, stream, ahead, ahead_blocks); break;
    case 8: launch_rank<8>(plan, ids, k, num_experts, align, expand_idx, hist, bflags, counts,
                           send, status, map, ranks, stream, ahead, ahead_blocks); break;
    default: launch_rank<16>(plan, ids, k, num_experts, align, expand_idx, hist, bflags, counts,
                             send, status, map, ranks, stream, ahead, ahead_blocks); break;
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || plan.blocks <= 1) return err;
  // The finalize pass looks pairs up by the id they were ranked under.
  const int32_t* ranked_ids = map.offsets != nullptr ? map.out : ids;
  launch_kernel(layout_finalize_kernel, plan.blocks + ahead_blocks, kLayoutThreads, stream,
      ranked_ids, (int32_t)plan.n_pairs, num_experts, align, (int32_t)plan.pairs_per_block,
      plan.blocks, hist, bflags, expand_idx, counts, send, status, ranks, ahead, ahead_blocks);
  return hipGetLastError();
}

}  // namespace moe
