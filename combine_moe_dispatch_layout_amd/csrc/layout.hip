// layout.hip -- routing -> per-expert counts, 128-padded exclusive prefix sum
// and stable within-expert ranks (the expert_ids / expand_idx /
// ep_send_counts triple of the npu_moe_distribute_combine page; the padding
// is the grouped GEMM's 128-row M-tile from the TEMPO summary, section 1).
//
// Ranking pass (one or more workgroups of 8 waves, at most kLayoutMaxBlocks):
//   A workgroup owns a contiguous range of whole tokens and walks it in
//   chunks of at most 2048 pairs.  Within a chunk, wave w owns a contiguous
//   run of 64*R pairs and walks it in R sub-rounds of 64 (one pair per lane),
//   entirely against its own LDS slice, so no workgroup barrier is needed
//   inside the walk:
//     - every lane ORs its bit into mask[w][e] for its expert e (LDS atomic
//       OR: the result does not depend on the order the lanes arrive in);
//     - a lane's local rank = wave_run[w][e] (pairs of e in this wave's
//       earlier sub-rounds) + popcount(mask & lanes below it);
//     - the lowest lane of each expert group advances wave_run[w][e] and
//       clears the mask word.
//   LDS instructions of one wave execute in issue order, so each step sees
//   the previous one.  After a workgroup barrier a per-expert exclusive
//   prefix over the 8 waves, started from the counts of the workgroup's
//   earlier chunks, turns local ranks into ranks within the workgroup.
//   Nothing positional is decided by an atomic race, so the layout is
//   deterministic.
// Repeated ids: when K divides the wave, each 64-pair sub-round holds whole
//   tokens, so a repeat is a second bit among the token's K lanes in the
//   expert's mask; otherwise (and for logical repeats under a replica map)
//   the chunk's ids are staged in LDS and each thread compares one token's
//   K ids in registers.
// Single workgroup (<= 2048 pairs): the same kernel also writes the counts and
//   the padded exclusive scan, so small batches take one launch.
// Several workgroups: each writes its expert histogram to the workspace,
//   publishes it (device-scope fence) and counts itself in on an arrival
//   counter.  The workgroup that arrives last sees every histogram: it turns
//   the histograms, in place, into the exclusive prefix over workgroups of
//   each expert's column (the device-wide scan, each column scanned once),
//   writes the counts, the padded scan and the status word, and sets the
//   counter back to zero for the next call.  Nobody waits for anybody.  The
//   ranks then need their workgroup's column prefix added: by a second, short
//   launch (moe_dispatch_layout), or by the scatter itself when the layout is
//   followed by one (moe_dispatch_fused).
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

// Flags an expert (an id in [0, E)) repeated within one of the chunk's
// tokens, from the chunk's ids staged in LDS (`chunk_ids[i]` = id of the
// chunk's pair i; the chunk holds whole tokens).  One token per thread, its
// K ids compared in registers.
__device__ __forceinline__ int duplicate_flags(const int* chunk_ids, int32_t n, int32_t k,
                                               int32_t E) {
  int fl = 0;
  for (int base = (int)threadIdx.x * k; base < n; base += kLayoutThreads * k) {
    int v[kMaxTopK];
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) v[j] = (j < k) ? chunk_ids[base + j] : -1 - j;
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

// Loads / stores W adjacent histogram columns (W = 4: one 16-byte access).
template <int W>
__device__ __forceinline__ void load_cols(const int32_t* p, int (&v)[W]) {
  if constexpr (W == 4) {
    const u32x4 q = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int w = 0; w < 4; ++w) v[w] = (int)q[w];
  } else {
    v[0] = *p;
  }
}
template <int W>
__device__ __forceinline__ void store_cols(int32_t* p, const int (&v)[W]) {
  if constexpr (W == 4) {
    *reinterpret_cast<u32x4*>(p) = u32x4{(uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2],
                                         (uint32_t)v[3]};
  } else {
    *p = v[0];
  }
}

// Each expert's column of the workgroup histograms ws.hist[b*E + e] is
// scanned once, in place, into the exclusive prefix over workgroups
// (workgroup b's first rank for that expert); totals[e] receives the column
// sum, the expert's count.  Threads own W adjacent columns (W = 4 when E is a
// multiple of 4, so every access is 16 bytes) and a run of rows, loaded in
// batches of kScanBatch accesses in flight.  A run of at most kScanKeep rows
// stays in registers between the two passes; a longer one is read again in
// the second pass.  `part` is LDS scratch of W * kLayoutThreads ints.
constexpr int kScanBatch = 16;
template <int W>
__device__ __forceinline__ void scan_columns(const LayoutScratch& ws, int32_t blocks, int32_t E,
                                             int* part, int* totals) {
  constexpr int kScanKeep = 16 / W;
  const int tid = threadIdx.x;
  const int ncol = E / W;
  int cpad = 1;
  while (cpad < ncol) cpad <<= 1;
  const int groups = kLayoutThreads / cpad;  // threads per column group, each a run of rows
  const int col = tid & (cpad - 1);
  const int grp = tid / cpad;
  const int rows = (blocks + groups - 1) / groups;
  const int r0 = min(blocks, grp * rows), r1 = min(blocks, r0 + rows);
  const bool active = col < ncol;
  const bool keep = r1 - r0 <= kScanKeep;
  int32_t* __restrict__ h = ws.hist + col * W;

  // Pass 1: this thread's partial column sums.
  int partial[W];
#pragma unroll
  for (int w = 0; w < W; ++w) partial[w] = 0;
  int kept[kScanKeep][W];
  if (active && keep) {
#pragma unroll
    for (int u = 0; u < kScanKeep; ++u) {
      if (r0 + u < r1) {
        load_cols<W>(h + (int64_t)(r0 + u) * E, kept[u]);
      } else {
#pragma unroll
        for (int w = 0; w < W; ++w) kept[u][w] = 0;
      }
    }
#pragma unroll
    for (int u = 0; u < kScanKeep; ++u)
#pragma unroll
      for (int w = 0; w < W; ++w) partial[w] += kept[u][w];
  } else if (active) {
    for (int b0 = r0; b0 < r1; b0 += kScanBatch) {
      int v[kScanBatch][W];
#pragma unroll
      for (int u = 0; u < kScanBatch; ++u) {
        if (b0 + u < r1) {
          load_cols<W>(h + (int64_t)(b0 + u) * E, v[u]);
        } else {
#pragma unroll
          for (int w = 0; w < W; ++w) v[u][w] = 0;
        }
      }
#pragma unroll
      for (int u = 0; u < kScanBatch; ++u)
#pragma unroll
        for (int w = 0; w < W; ++w) partial[w] += v[u][w];
    }
  }
#pragma unroll
  for (int w = 0; w < W; ++w) part[w * kLayoutThreads + tid] = partial[w];
  __syncthreads();
  int run[W], total[W];
#pragma unroll
  for (int w = 0; w < W; ++w) {
    run[w] = 0;
    total[w] = 0;
    for (int g = 0; g < groups; ++g) {
      const int p = part[w * kLayoutThreads + g * cpad + col];
      run[w] += (g < grp) ? p : 0;
      total[w] += p;
    }
  }
  // Pass 2: the exclusive prefix down the columns, written over the counts.
  if (active && keep) {
#pragma unroll
    for (int u = 0; u < kScanKeep; ++u) {
      if (r0 + u < r1) {
        store_cols<W>(h + (int64_t)(r0 + u) * E, run);
#pragma unroll
        for (int w = 0; w < W; ++w) run[w] += kept[u][w];
      }
    }
  } else if (active) {
    for (int b0 = r0; b0 < r1; b0 += kScanBatch) {
      int v[kScanBatch][W];
#pragma unroll
      for (int u = 0; u < kScanBatch; ++u) {
        if (b0 + u < r1) {
          load_cols<W>(h + (int64_t)(b0 + u) * E, v[u]);
        } else {
#pragma unroll
          for (int w = 0; w < W; ++w) v[u][w] = 0;
        }
      }
#pragma unroll
      for (int u = 0; u < kScanBatch; ++u) {
        if (b0 + u < r1) {
          store_cols<W>(h + (int64_t)(b0 + u) * E, run);
#pragma unroll
          for (int w = 0; w < W; ++w) run[w] += v[u][w];
        }
      }
    }
  }
  if (active && grp == 0) {
#pragma unroll
    for (int w = 0; w < W; ++w) totals[col * W + w] = total[w];
  }
}

// Run by the workgroup that arrived last, after its acquire fence: every
// workgroup's histogram row is in ws.hist[b*E + e].  The columns are scanned
// (scan_columns), then the padded scan of the totals gives the offsets.
// `part` is LDS scratch of at least 5 * kLayoutThreads ints.
__device__ void finish_layout(const LayoutScratch& ws, int32_t blocks, int32_t E, int32_t align,
                              int* part, int* wave_tot, int* flags_lds,
                              int32_t* __restrict__ counts, int32_t* __restrict__ send,
                              int32_t* __restrict__ status, const RankSplit& ranks) {
  const int tid = threadIdx.x;
  // Each workgroup's flag word is one thread's (at most kLayoutMaxBlocks <
  // kLayoutThreads workgroups); its load is issued before the columns'.
  static_assert(kLayoutMaxBlocks <= kLayoutThreads, "one flag word per thread");
  const int f = (tid < blocks) ? ws.flags[tid] : 0;
  int* totals = part + 4 * kLayoutThreads;
  if ((E & 3) == 0)
    scan_columns<4>(ws, blocks, E, part, totals);
  else
    scan_columns<1>(ws, blocks, E, part, totals);
  if (f) atomicOr(flags_lds, f);
  __syncthreads();
  write_counts_and_offsets(tid < E ? totals[tid] : 0, E, align, wave_tot, counts, send, ranks);
  if (tid == 0) {
    if (status) *status = *flags_lds;
    atomicExch(ws.arrivals, 0);  // ready for the next call
  }
}

// Ranking over E "experts".  With a replica map, ids are logical experts in
// [0, map.n_logical) and each pair is first sent to one of its expert's
// physical replicas (E = number of replicas): u = upper 32 bits of the pair's
// SplitMix64 draw, replica = first r of the expert's range with
// u <= thresholds[r] (TEMPO summary, section 2: probabilistic replica
// dispatch and count gathering in one in-graph kernel).
// Workgroups past rank_blocks read the token rows ahead instead.  MAPPED
// (a replica map is given) is a template parameter, so that the plain
// ranking carries none of the mapping's code and registers.
template <int R, bool MAPPED>
__global__ __launch_bounds__(kLayoutThreads) void layout_rank_kernel(
    const int32_t* __restrict__ ids, int32_t n_pairs, int32_t k, int32_t E, int32_t align,
    int32_t chunk_pairs, int32_t chunks, int32_t* __restrict__ ranks_out, LayoutScratch ws,
    int32_t* __restrict__ counts, int32_t* __restrict__ send, int32_t* __restrict__ status,
    ReplicaMap map, RankSplit ranks, ReadAhead ahead, int32_t rank_blocks,
    int32_t ahead_blocks) {
  if ((int32_t)blockIdx.x >= rank_blocks) {
    read_ahead(ahead, rank_blocks, ahead_blocks, 0, ahead.vecs);
    return;
  }
  __shared__ unsigned long long mask[kLayoutWaves][kMaxExperts];  // 32 KB
  __shared__ int wave_run[kLayoutWaves][kMaxExperts];             // 16 KB
  __shared__ int chunk_ids[kLayoutThreads * R];  // the chunk's input ids, for repeats
  __shared__ int blk_run[kMaxExperts];   // pairs per expert in earlier chunks
  __shared__ int rep_off[kMaxExperts + 1];
  __shared__ uint32_t rep_thr[kMaxExperts];
  __shared__ int wave_tot[kLayoutWaves];
  __shared__ int flags_lds;
  __shared__ int last_lds;
  constexpr bool mapped = MAPPED;
  const int32_t n_ids = mapped ? map.n_logical : E;  // valid range of the input ids

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int64_t ppb = (int64_t)chunk_pairs * chunks;
  const int64_t bbegin = (int64_t)blockIdx.x * ppb;
  const int64_t bend = min((int64_t)n_pairs, bbegin + ppb);

  // The first chunk's id loads are issued before the LDS set-up, and under
  // a replica map so are the tables' loads (at most n_ids + 1 <= 513
  // offsets and E <= 512 thresholds: two and one per thread) and the first
  // chunk's draws, which depend on the pair index only.
  int e[R];
  uint32_t u0[R];
  {
    const int64_t end = min(bend, bbegin + chunk_pairs);
    const int64_t wbase = bbegin + wave * (kWave * R);
#pragma unroll
    for (int s = 0; s < R; ++s) {
      const int64_t i = wbase + s * kWave + lane;
      e[s] = (i < end) ? ids[i] : 0;
    }
  }
  static_assert(kMaxExperts + 1 <= 2 * kLayoutThreads && kMaxExperts <= kLayoutThreads,
                "replica tables: two offsets and one threshold per thread");
  int off_a = 0, off_b = 0;
  uint32_t thr_a = 0;
  if (mapped) {
    if (tid <= n_ids) off_a = map.offsets[tid];
    if (tid + kLayoutThreads <= n_ids) off_b = map.offsets[tid + kLayoutThreads];
    if (tid < E) thr_a = map.thresholds[tid];
    const int64_t wbase = bbegin + wave * (kWave * R);
#pragma unroll
    for (int s = 0; s < R; ++s)
      u0[s] = (uint32_t)(splitmix64(map.seed, (uint64_t)(wbase + s * kWave + lane)) >> 32);
  }

  for (int j = tid; j < kLayoutWaves * kMaxExperts; j += kLayoutThreads) {
    (&mask[0][0])[j] = 0ull;
    (&wave_run[0][0])[j] = 0;
  }
  for (int j = tid; j < kMaxExperts; j += kLayoutThreads) blk_run[j] = 0;
  if (tid == 0) flags_lds = 0;
  if (mapped) {
    if (tid <= n_ids) rep_off[tid] = off_a;
    if (tid + kLayoutThreads <= n_ids) rep_off[tid + kLayoutThreads] = off_b;
    if (tid < E) rep_thr[tid] = thr_a;
  }
  int fl = 0;
  __syncthreads();

  const unsigned long long below_me = (1ull << lane) - 1ull;
  // Repeated experts within a token: when K divides the wave, every chunk's
  // 64-pair sub-rounds hold whole tokens, so a repeat shows in the expert's
  // lane mask as a second bit among the token's K lanes; under a replica map
  // (repeats are of logical experts, which the masks no longer see) each
  // lane compares its id with the token's earlier lanes' by cross-lane
  // shuffles instead.  Otherwise the chunk's ids are staged in LDS and each
  // token's K ids compared.
  const bool whole_tokens = kWave % k == 0;
  const bool mask_dups = !mapped && whole_tokens;
  const bool shuffle_dups = mapped && whole_tokens;
  const unsigned long long token_lanes =
      (k >= kWave ? ~0ull : ((1ull << k) - 1ull)) << (lane - lane % k);
  for (int c = 0; c < chunks; ++c) {
    const int64_t begin = bbegin + (int64_t)c * chunk_pairs;
    if (begin >= bend) break;  // workgroup-uniform
    const int64_t end = min(bend, begin + chunk_pairs);
    const int64_t wbase = begin + wave * (kWave * R);
    if (c > 0) {
#pragma unroll
      for (int s = 0; s < R; ++s) {
        const int64_t i = wbase + s * kWave + lane;
        e[s] = (i < end) ? ids[i] : 0;
      }
    }
    if (!whole_tokens) {
#pragma unroll
      for (int s = 0; s < R; ++s) {
        const int64_t i = wbase + s * kWave + lane;
        if (i < end) chunk_ids[i - begin] = e[s];  // as given, before any replica mapping
      }
    }
    if (shuffle_dups) {
      // Lane pos of a token against each earlier lane of it, the R
      // sub-rounds' shuffles of one distance issued together.
      const int pos = lane % k;  // this pair's place in its token
      bool valid[R];
#pragma unroll
      for (int s = 0; s < R; ++s) {
        const int64_t i = wbase + s * kWave + lane;
        valid[s] = i < end && e[s] >= 0 && e[s] < n_ids;
      }
      for (int d = 1; d < k; ++d) {
        int other[R];
#pragma unroll
        for (int s = 0; s < R; ++s) other[s] = __shfl_up(e[s], d, kWave);
#pragma unroll
        for (int s = 0; s < R; ++s)
          if (valid[s] && pos >= d && other[s] == e[s]) fl |= MOE_FLAG_DUP_ID;
      }
    }

    if (mapped) {
      // Replica r of pair i: the first q of its expert's range (clipped to
      // [0, E)) with u <= thresholds[q].  The R pairs' table lookups go
      // side by side rather than one pair's whole search after another's.
      int lo[R], hi[R], r[R];
      uint32_t u[R];
      int steps = 0;
#pragma unroll
      for (int s = 0; s < R; ++s) {
        const int64_t i = wbase + s * kWave + lane;
        const bool valid = i < end && e[s] >= 0 && e[s] < n_ids;
        if (i < end && !valid) fl |= MOE_FLAG_ID_RANGE;
        lo[s] = valid ? max(rep_off[e[s]], 0) : 0;
        hi[s] = valid ? min(rep_off[e[s] + 1], E) : 0;
        u[s] = c == 0 ? u0[s] : (uint32_t)(splitmix64(map.seed, (uint64_t)i) >> 32);
        r[s] = -1;
        steps = max(steps, hi[s] - lo[s]);
      }
      // The first kFirstSteps entries of every range in one round of reads
      // (read unconditionally, the index kept in range, so that they all go
      // out together); longer ranges continue one step at a time.
      constexpr int kFirstSteps = 4;
      {
        uint32_t thr[R][kFirstSteps];
#pragma unroll
        for (int s = 0; s < R; ++s)
#pragma unroll
          for (int d = 0; d < kFirstSteps; ++d) thr[s][d] = rep_thr[min(lo[s] + d, E - 1)];
#pragma unroll
        for (int s = 0; s < R; ++s)
#pragma unroll
          for (int d = 0; d < kFirstSteps; ++d) {
            const int q = lo[s] + d;
            if (r[s] < 0 && q < hi[s] && u[s] <= thr[s][d]) r[s] = q;
          }
      }
      for (int d = kFirstSteps; d < steps; ++d) {
        uint32_t thr[R];
#pragma unroll
        for (int s = 0; s < R; ++s) thr[s] = rep_thr[min(lo[s] + d, E - 1)];
#pragma unroll
        for (int s = 0; s < R; ++s) {
          const int q = lo[s] + d;
          if (r[s] < 0 && q < hi[s] && u[s] <= thr[s]) r[s] = q;
        }
      }
#pragma unroll
      for (int s = 0; s < R; ++s) {
        const int64_t i = wbase + s * kWave + lane;
        if (i >= end) continue;
        if (r[s] < 0 && e[s] >= 0 && e[s] < n_ids) fl |= MOE_FLAG_REPLICA;
        map.out[i] = r[s];
        e[s] = r[s];  // ranked as a physical replica; -1 drops the pair
      }
    }

    int lr[R];
#pragma unroll
    for (int s = 0; s < R; ++s) {
      const int64_t i = wbase + s * kWave + lane;
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
      if (mask_dups && ok && __popcll(m & token_lanes) > 1) fl |= MOE_FLAG_DUP_ID;
      lr[s] = ok ? before + below : -1;
      if (ok && below == 0) {
        wave_run[wave][e[s]] = before + __popcll(m);
        mask[wave][e[s]] = 0ull;
      }
      __builtin_amdgcn_wave_barrier();
    }
    __syncthreads();
    if (!whole_tokens) fl |= duplicate_flags(chunk_ids, (int32_t)(end - begin), k, n_ids);

    // Exclusive prefix over waves, per expert, after the earlier chunks.
    int run = 0;
    if (tid < E) {
      run = blk_run[tid];
#pragma unroll
      for (int w = 0; w < kLayoutWaves; ++w) {
        const int cnt = wave_run[w][tid];
        wave_run[w][tid] = run;
        run += cnt;
      }
    }
    __syncthreads();

#pragma unroll
    for (int s = 0; s < R; ++s) {
      const int64_t i = wbase + s * kWave + lane;
      if (i < end) ranks_out[i] = lr[s] >= 0 ? lr[s] + wave_run[wave][e[s]] : -1;
    }
    if (tid < E) blk_run[tid] = run;  // read back below only by the same thread
    if (end < bend) {  // another chunk follows (workgroup-uniform)
      __syncthreads();
      if (tid < E) {
#pragma unroll
        for (int w = 0; w < kLayoutWaves; ++w) wave_run[w][tid] = 0;
      }
      __syncthreads();
    }
  }
  if (fl) atomicOr(&flags_lds, fl);
  __syncthreads();
  const int tot = tid < E ? blk_run[tid] : 0;

  if (ws.hist == nullptr) {
    // The whole batch was this workgroup: finish the layout here.
    write_counts_and_offsets(tot, E, align, wave_tot, counts, send, ranks);
    if (tid == 0 && status) *status = flags_lds;
    return;
  }
  if (tid < E) ws.hist[(int64_t)blockIdx.x * E + tid] = tot;
  if (tid == 0) ws.flags[blockIdx.x] = flags_lds;
  // Count in with a device-scope release: after the workgroup barrier, one
  // wave's release (an L2 write-back on this multi-XCD device) publishes
  // every wave's writes before the increment.
  __syncthreads();
  if (tid == 0) {
    const int before = __hip_atomic_fetch_add(ws.arrivals, 1, __ATOMIC_RELEASE,
                                              __HIP_MEMORY_SCOPE_AGENT);
    last_lds = (before == rank_blocks - 1) ? 1 : 0;
    if (last_lds) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // the other histograms
      flags_lds = 0;
    }
  }
  __syncthreads();
  if (!last_lds) return;
  finish_layout(ws, rank_blocks, E, align, &wave_run[0][0], wave_tot, &flags_lds, counts, send,
                status, ranks);
}

// Adds each workgroup's column prefix (from the arrival-ordered scan) to the
// ranks within that workgroup.  One workgroup per ranking workgroup.
__global__ __launch_bounds__(kLayoutThreads) void layout_finalize_kernel(
    const int32_t* __restrict__ ids, int32_t n_pairs, int32_t E, int64_t pairs_per_block,
    const int32_t* __restrict__ base, int32_t* __restrict__ expand_idx) {
  __shared__ int base_lds[kMaxExperts];
  constexpr int kUnroll = 4;
  const int tid = threadIdx.x;
  const int64_t begin = (int64_t)blockIdx.x * pairs_per_block;
  const int64_t end = min((int64_t)n_pairs, begin + pairs_per_block);
  bool staged = false;
  for (int64_t i0 = begin; i0 < end; i0 += kUnroll * kLayoutThreads) {
    int r[kUnroll], e[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = i0 + u * kLayoutThreads + tid;
      r[u] = (i < end) ? expand_idx[i] : -1;
      e[u] = (i < end) ? ids[i] : 0;
    }
    if (!staged) {  // workgroup-uniform; overlaps the first loads
      for (int j = tid; j < E; j += kLayoutThreads) base_lds[j] = base[blockIdx.x * E + j];
      __syncthreads();
      staged = true;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = i0 + u * kLayoutThreads + tid;
      if (r[u] >= 0) expand_idx[i] = r[u] + base_lds[e[u]];
    }
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
    p.chunk_pairs = (int32_t)p.n_pairs;
    p.chunks = 1;
  } else {
    // Chunks of whole tokens, so that every token lies in one workgroup.
    p.rounds = kLayoutMultiRounds;
    p.chunk_pairs = (kLayoutThreads * kLayoutMultiRounds / k) * k;
    const int64_t total_chunks = (p.n_pairs + p.chunk_pairs - 1) / p.chunk_pairs;
    p.chunks = (int32_t)((total_chunks + kLayoutMaxBlocks - 1) / kLayoutMaxBlocks);
    const int64_t ppb = (int64_t)p.chunks * p.chunk_pairs;
    p.blocks = (int32_t)((p.n_pairs + ppb - 1) / ppb);
  }
  p.pairs_per_block = (int64_t)p.chunks * p.chunk_pairs;
  return p;
}

namespace {

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

}  // namespace

// Workspace layout: the arrival counter in the first 256 bytes, at the same
// place for every shape (so a workspace reused for batches of other shapes
// still holds a zero counter there), then the histograms, the flags and the
// ranks within the workgroups.
constexpr size_t kCounterBytes = 256;

size_t layout_workspace_bytes(const LayoutPlan& p, int32_t num_experts) {
  if (p.blocks <= 1) return 0;
  return kCounterBytes + align256((size_t)p.blocks * num_experts * sizeof(int32_t)) +
         align256((size_t)p.blocks * sizeof(int32_t)) +
         align256((size_t)p.n_pairs * sizeof(int32_t));
}

LayoutScratch layout_scratch(const LayoutPlan& p, int32_t num_experts, void* workspace) {
  LayoutScratch ws;
  if (p.blocks <= 1) return ws;
  char* base = static_cast<char*>(workspace);
  const size_t hist = align256((size_t)p.blocks * num_experts * sizeof(int32_t));
  const size_t flags = align256((size_t)p.blocks * sizeof(int32_t));
  ws.arrivals = reinterpret_cast<int32_t*>(base);
  ws.hist = reinterpret_cast<int32_t*>(base + kCounterBytes);
  ws.flags = reinterpret_cast<int32_t*>(base + kCounterBytes + hist);
  ws.ranks = reinterpret_cast<int32_t*>(base + kCounterBytes + hist + flags);
  return ws;
}

namespace {

template <int R>
void launch_rank(const LayoutPlan& plan, const int32_t* ids, int32_t k, int32_t E, int32_t align,
                 int32_t* ranks_out, const LayoutScratch& ws, int32_t* counts, int32_t* send,
                 int32_t* status, const ReplicaMap& map, const RankSplit& ranks,
                 hipStream_t stream, const ReadAhead& ahead, int32_t ahead_blocks) {
  if (map.offsets != nullptr)
    launch_kernel(layout_rank_kernel<R, true>, plan.blocks + ahead_blocks, kLayoutThreads,
        stream, ids, (int32_t)plan.n_pairs, k, E, align, plan.chunk_pairs, plan.chunks,
        ranks_out, ws, counts, send, status, map, ranks, ahead, plan.blocks, ahead_blocks);
  else
    launch_kernel(layout_rank_kernel<R, false>, plan.blocks + ahead_blocks, kLayoutThreads,
        stream, ids, (int32_t)plan.n_pairs, k, E, align, plan.chunk_pairs, plan.chunks,
        ranks_out, ws, counts, send, status, map, ranks, ahead, plan.blocks, ahead_blocks);
}

}  // namespace

namespace {

// The read-ahead workgroups alone, for a scatter with no layout launch before
// it (moe_dispatch).
__global__ __launch_bounds__(kLayoutThreads) void read_ahead_kernel(ReadAhead ahead) {
  read_ahead(ahead, 0, (int32_t)gridDim.x, 0, ahead.vecs);
}

}  // namespace

hipError_t launch_read_ahead(const ReadAhead& ahead, hipStream_t stream) {
  launch_kernel(read_ahead_kernel, kReadAheadMaxBlocks, kLayoutThreads, stream, ahead);
  return hipGetLastError();
}

hipError_t launch_layout(const int32_t* ids, int32_t k, int32_t num_experts, int32_t align,
                         const LayoutPlan& plan, int32_t* counts, int32_t* send,
                         int32_t* expand_idx, int32_t* status, void* workspace,
                         const ReplicaMap& map, const RankSplit& ranks, hipStream_t stream,
                         const ReadAhead& ahead, bool defer_ranks) {
  const int32_t ahead_blocks =
      read_ahead_runs(plan, ahead) ? kReadAheadMaxBlocks - plan.blocks : 0;
  const LayoutScratch ws = layout_scratch(plan, num_experts, workspace);
  // With several workgroups and a scatter to follow, the ranks within the
  // workgroups stay in the workspace and the scatter completes expand_idx.
  int32_t* ranks_out = (plan.blocks > 1 && defer_ranks) ? ws.ranks : expand_idx;
  switch (plan.rounds) {
    case 1: launch_rank<1>(plan, ids, k, num_experts, align, ranks_out, ws, counts, send,
                           status, map, ranks, stream, ahead, ahead_blocks); break;
    case 2: launch_rank<2>(plan, ids, k, num_experts, align, ranks_out, ws, counts, send,
                           status, map, ranks, stream, ahead, ahead_blocks); break;
    default: launch_rank<4>(plan, ids, k, num_experts, align, ranks_out, ws, counts, send,
                            status, map, ranks, stream, ahead, ahead_blocks); break;
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || plan.blocks <= 1 || defer_ranks) return err;
  // The finalize pass looks pairs up by the id they were ranked under.
  const int32_t* ranked_ids = map.offsets != nullptr ? map.out : ids;
  launch_kernel(layout_finalize_kernel, plan.blocks, kLayoutThreads, stream, ranked_ids,
      (int32_t)plan.n_pairs, num_experts, plan.pairs_per_block, (const int32_t*)ws.hist,
      expand_idx);
  return hipGetLastError();
}

}  // namespace moe
