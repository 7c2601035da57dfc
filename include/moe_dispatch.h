/*
 * moe_dispatch.h -- C ABI of the MI355X (gfx950) MoE token dispatch / combine
 * library (libmoe_dispatch.so).
 *
 * The three entry points are the local (one-device) stages of the pair of
 * operators documented on the torch_npu API reference page for
 * npu_moe_distribute_combine (Ascend): the dispatch side lays token rows out
 * expert-contiguously and returns expand_idx and the send counts in
 * prefix-sum form; the combine side retraces that path back to token order
 * and forms the weighted sum of the formula in that page's 计算公式 (formula)
 * section.
 * With one device the page's ReduceScatterV (tensor-parallel) and AlltoAllv
 * (expert-parallel) exchanges are identities: the whole expert set is the one
 * expert-parallel rank's share.
 *
 * Conventions for every call:
 *  - Tensor pointers are DEVICE pointers owned by the caller (for example
 *    allocated by PyTorch).  The library allocates nothing, keeps no state
 *    between calls (apart from the per-thread timing events of
 *    moe_time_next_launches in moe_probe.h, a measurement aid) and is safe
 *    to call from several host threads.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  A
 *    call validates its arguments on the host, enqueues its kernels on
 *    `stream` and returns; it never synchronises.  Buffers must stay alive
 *    and unmodified until the stream has finished the call (the page on the
 *    DeepSeek Ascend toolchain, troubleshooting step 5: reuse or free buffers
 *    only after the asynchronous work is done).
 *  - Row strides are counted in elements of the row's own type.
 *  - A failed argument check returns a non-zero moe_status and enqueues
 *    nothing.  Problems that only the device can see (ids out of range,
 *    repeated ids, a slot beyond the buffer) set bits of the optional
 *    device-side `status` word and the offending pair is skipped; no write
 *    ever leaves the caller's buffers (the DeepEP compensation PR, Kernel /
 *    host section: fail-safe bounds guards on the scatter writes).
 *  - No call waits on another device (same toolchain page, single-card
 *    compute section: a local operator never holds a cross-rank wait).
 */
#ifndef MOE_DISPATCH_H
#define MOE_DISPATCH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
enum moe_status {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1,   /* a shape, range, pointer or alignment rule failed */
    MOE_ERR_WORKSPACE = 2,     /* workspace_bytes below moe_dispatch_layout_workspace_size */
    MOE_ERR_UNSUPPORTED = 3,   /* unknown dtype */
    MOE_ERR_HIP = 4,           /* the HIP runtime refused a launch */
    MOE_ERR_SCRATCH = 5        /* batch too large for moe_dispatch_fused_noalloc's scratch */
};

/* Element type of the dispatched buffer. */
enum moe_dtype {
    MOE_BF16 = 0,              /* bfloat16 bit copy of the token row */
    MOE_FP8_E4M3 = 1           /* OCP e4m3fn (max 448) + one fp32 scale per 128 channels */
};

/* Bits of the device-side status word. */
enum moe_flag {
    MOE_FLAG_ID_RANGE = 1,     /* some expert_ids value lies outside [0, num_experts) */
    MOE_FLAG_DUP_ID = 2,       /* some row of expert_ids repeats an expert */
    MOE_FLAG_GUARD = 4,        /* some slot fell outside [0, capacity_rows): pair skipped */
    MOE_FLAG_REPLICA = 8       /* a replica table gave an expert no replica for some draw */
};

/* Version of this interface (incremented on any change of a signature or of
 * a caller's obligations; 2: the layout workspace must start zero-filled). */
int moe_abi_version(void);

/* Human-readable text of a moe_status value (static storage). */
const char* moe_status_string(int status);

/*
 * Rows of the expert-contiguous buffer that always hold the padded layout,
 * whatever the routing: with n = bs*k pairs, each expert's segment is rounded
 * up to a multiple of `align`, so the total is at most
 *   align * floor((n + (align-1) * min(num_experts, n)) / align).
 * This is the padded form of the page's rule that A, the number of rows a
 * card receives, be at least BS * min(local_expert_num, K) per source card
 * (npu_moe_distribute_combine, constraint notes on A).  Returns -1 when the
 * arguments break the rules of moe_dispatch_layout.
 */
int64_t moe_dispatch_capacity(int32_t bs, int32_t k, int32_t num_experts, int32_t align);

/* Bytes of device workspace moe_dispatch_layout (and the fused and
 * replica-aware calls) need for this shape: 0 when the whole layout fits one
 * workgroup (bs*k <= 2048; then `workspace` may be NULL).  Returns 0 for
 * invalid arguments as well; the layout call reports those.
 * The workspace must be zero-filled before its first use (for example with
 * hipMemset, or a fill kernel where a memset node is unwanted, as under
 * graph capture).  Its first word is an arrival counter that tells a ranking
 * workgroup it is the last to finish; every call leaves that word zero
 * again, so one workspace serves any number of calls of any shapes that fit
 * it, one call at a time.  The rest (the ranking workgroups' histograms,
 * which the last workgroup scans, their flags and ranks) needs no initial
 * contents. */
size_t moe_dispatch_layout_workspace_size(int32_t bs, int32_t k, int32_t num_experts);

/*
 * Layout: routing -> per-expert counts, padded prefix sum, stable ranks.
 *
 * Follows the parameters expert_ids, expand_idx and ep_send_counts of the
 * npu_moe_distribute_combine page (which are the paired dispatch operator's
 * outputs) and the 128-row M-tile padding of the grouped GEMM in the TEMPO
 * summary (section 1, padded compute).
 *
 *  expert_ids     in  int32 [bs, k], row-major, contiguous.  Values must lie in
 *                     [0, num_experts) and be distinct within a row (page rule).
 *  bs             in  tokens, >= 0 (0 is an empty batch: counts and offsets 0).
 *  k              in  experts per token, 1 <= k <= min(16, num_experts).
 *  num_experts    in  1 <= num_experts <= 512.
 *  align          in  segment alignment in rows, a power of two in [1, 1024];
 *                     128 matches the grouped GEMM's M-tile.
 *  expert_counts  out int32 [num_experts]: c_e = number of pairs routed to e.
 *  ep_send_counts out int32 [num_experts + 1]: exclusive prefix of the padded
 *                     counts ceil(c_e/align)*align; entry num_experts is the
 *                     padded total M_pad.  Every entry is a multiple of align.
 *  expand_idx     out int32 [bs * k]: for pair (t, j), the number of pairs
 *                     (t', j') before it in row-major order routed to the same
 *                     expert (the within-expert rank), or -1 if its id is out
 *                     of range.  Pair (t, j) lives in row
 *                     ep_send_counts[expert_ids[t,j]] + expand_idx[t*k+j].
 *  status         out int32 [1] or NULL: OR of MOE_FLAG_ID_RANGE and
 *                     MOE_FLAG_DUP_ID, overwritten (not accumulated).
 *                     Out-of-range pairs are excluded from the counts;
 *                     repeated ids are laid out like distinct ones.
 *  workspace      in/out device scratch of workspace_bytes >=
 *                     moe_dispatch_layout_workspace_size(bs, k, num_experts),
 *                     16-byte aligned, zero-filled before its first use (see
 *                     moe_dispatch_layout_workspace_size); calls that share a
 *                     workspace must not overlap.
 * The result is deterministic (no atomics decide any position).  Batches of
 * more than 2048 pairs take two launches: ranking workgroups of whole tokens
 * (at most 256, each walking chunks of at most 2048 pairs) write their
 * ranks and per-expert histograms, and the last of them to finish turns the
 * histograms into each expert's exclusive prefix over workgroups (a
 * device-wide scan in which every histogram entry is read and written once)
 * and writes the counts and ep_send_counts; a second launch adds each
 * workgroup's prefix to its ranks.  Work grows linearly with bs*k.
 */
int moe_dispatch_layout(const int32_t* expert_ids, int32_t bs, int32_t k, int32_t num_experts,
                        int32_t align, int32_t* expert_counts, int32_t* ep_send_counts,
                        int32_t* expand_idx, int32_t* status, void* workspace,
                        size_t workspace_bytes, void* stream);

/*
 * Rank-partitioned layout: moe_dispatch_layout plus the per-destination-rank
 * send offsets an expert-parallel all-to-all(v) needs.  The combine page's
 * A3-series ep_send_counts has ep_world_size * local_expert_num entries and
 * its expert count must divide evenly over the expert ranks: expert e lives
 * on rank e / L with L = num_experts / ep_world_size, so the expert-major
 * layout is already rank-major and rank r's rows are
 *   [rank_offsets[r], rank_offsets[r+1]),  rank_offsets[r] = ep_send_counts[r*L],
 * rank_offsets[ep_world_size] = the padded total.  With align = 1 the send
 * buffer carries no padding rows.
 *
 *  ep_world_size  in  1 <= ep_world_size <= num_experts, dividing num_experts.
 *  rank_offsets   out int32 [ep_world_size + 1].
 * Other arguments and outputs as for moe_dispatch_layout.
 */
int moe_dispatch_layout_ep(const int32_t* expert_ids, int32_t bs, int32_t k, int32_t num_experts,
                           int32_t ep_world_size, int32_t align, int32_t* expert_counts,
                           int32_t* ep_send_counts, int32_t* rank_offsets, int32_t* expand_idx,
                           int32_t* status, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * Replica-aware layout: the in-graph probabilistic dispatch with count
 * gathering of the TEMPO summary (section 2, system integration), where hot
 * experts have several physical replicas and each (token, k) pair is sent to
 * one of them.  Replicas of logical expert e are the physical ids
 * [replica_offsets[e], replica_offsets[e+1]), contiguous and disjoint.  Pair
 * i = t*k + j draws u = the upper 32 bits of draw i of the SplitMix64 stream
 * seeded with `seed` (Steele, Lea and Flood, OOPSLA 2014: the state
 * seed + (i+1)*0x9E3779B97F4A7C15 through the variant-13 finaliser), and
 * goes to the first replica r of its expert with u <= replica_thresholds[r]
 * (thresholds are cumulative within an expert; the last should be
 * 0xFFFFFFFF).  Then the layout of moe_dispatch_layout runs over the
 * num_replicas physical replicas: replica_counts[r] is the token count N_r
 * gathered per replica, ep_send_counts its 128-padded exclusive prefix (so
 * replica r spans ceil(N_r/128) M-tiles), expand_idx the stable rank.
 * Dispatch and combine then take replica_ids as their expert_ids with
 * num_experts = num_replicas.
 *
 *  expert_ids          in  int32 [bs, k] logical experts in [0, num_experts).
 *  replica_offsets     in  int32 [num_experts + 1], non-decreasing, last =
 *                          num_replicas (device memory).
 *  replica_thresholds  in  uint32 [num_replicas] (device memory).
 *  num_replicas        in  1 <= num_replicas <= 512, k <= num_replicas.
 *  replica_ids         out int32 [bs, k]: chosen replica, -1 if the logical id
 *                          is out of range (MOE_FLAG_ID_RANGE) or the table
 *                          gives none (MOE_FLAG_REPLICA); such pairs are
 *                          dropped like out-of-range ids.
 *  workspace           as for moe_dispatch_layout, sized with num_replicas.
 * Other arguments as for moe_dispatch_layout.  Deterministic for a fixed seed.
 */
int moe_dispatch_layout_replicated(const int32_t* expert_ids, int32_t bs, int32_t k,
                                   int32_t num_experts, const int32_t* replica_offsets,
                                   const uint32_t* replica_thresholds, int32_t num_replicas,
                                   uint64_t seed, int32_t align, int32_t* replica_ids,
                                   int32_t* replica_counts, int32_t* ep_send_counts,
                                   int32_t* expand_idx, int32_t* status, void* workspace,
                                   size_t workspace_bytes, void* stream);

/*
 * Dispatch: scatter token rows into the expert-contiguous buffer.
 *
 * The inverse path of the combine on the npu_moe_distribute_combine page
 * (function description: combine retraces the dispatch path); expand_x is
 * that page's (max(tp,1)*A, H) input, here [capacity_rows, hidden].  With
 * out_dtype MOE_FP8_E4M3 the rows are quantised on the way, the page's
 * comm_quant_mode option for a quantised transfer (its dtype is unreadable
 * on the page; e4m3fn with per-128-channel scales is this library's
 * reading).
 *
 *  x              in  bf16 [bs, hidden], row stride x_stride (>= hidden);
 *                     base 16-byte aligned, x_stride*2 a multiple of 16.
 *  hidden         in  > 0, a multiple of 32 (page rule on H), <= 65536;
 *                     a multiple of 128 for MOE_FP8_E4M3; bs*hidden/8 < 2^31.
 *  expert_ids, expand_idx, ep_send_counts
 *                 in  the layout call's input and outputs, unchanged.
 *  expand_x       out [capacity_rows, hidden] of out_dtype, row stride
 *                     expand_x_stride (>= hidden); 16-byte aligned, stride in
 *                     bytes a multiple of 16.  Row slot(t,j) receives token t
 *                     for every pair j.  Padding rows are NOT written.
 *  capacity_rows  in  rows of expand_x (size it with moe_dispatch_capacity).
 *                     A smaller value is accepted (a caller that knows the
 *                     padded total may size the buffer to it), but a pair
 *                     whose row lies at or beyond capacity_rows is DROPPED:
 *                     its row is not written and MOE_FLAG_GUARD is set in
 *                     `status`, which such a caller must read.  With 0 rows
 *                     every pair is guarded and nothing is written; expand_x
 *                     and quant_scales may then be NULL.
 *  quant_scales   out fp32 [capacity_rows, hidden/128] row-major when
 *                     out_dtype is MOE_FP8_E4M3 (else ignored, may be NULL):
 *                     s = amax/448 over the 128 channels of the block;
 *                     the code is e4m3(x/s) rounded to nearest even and
 *                     saturated to +-448 (all-zero block: s = 0, codes 0).
 *                     Dequantise as e4m3_value * s.
 *  status         in/out int32 [1] or NULL: MOE_FLAG_GUARD is OR-ed in when a
 *                     slot falls outside [0, capacity_rows); never cleared.
 *
 * Launches: one scatter; for bf16 output, when x is contiguous (x_stride ==
 * hidden) and its rows total 32 MB to 240 MB, a launch that reads them into
 * the 256 MB Infinity Cache goes first, so that the scatter writes from
 * cache-resident rows instead of interleaving row reads from HBM with its
 * writes.
 */
int moe_dispatch(const void* x, int64_t x_stride, int32_t bs, int32_t hidden,
                 const int32_t* expert_ids, const int32_t* expand_idx,
                 const int32_t* ep_send_counts, int32_t k, int32_t num_experts, void* expand_x,
                 int64_t expand_x_stride, int64_t capacity_rows, int32_t out_dtype,
                 float* quant_scales, int32_t* status, void* stream);

/*
 * Layout and dispatch in one call: the results of moe_dispatch_layout
 * followed by moe_dispatch on the same stream, bit for bit (outputs, padding
 * rows left unwritten, e4m3 codes and scales, status bits).  For
 * decode-sized batches (bs*k <= 2048) it is a single kernel launch: every
 * scatter workgroup derives the whole layout from the ids in on-chip memory,
 * so no separate layout launch or wait precedes the scatter (the TEMPO
 * summary, section 2, folds count gathering into the dispatch kernel; here
 * the counts, offsets and ranks are folded in).  Larger batches take two
 * launches: the layout's ranking launch (its last workgroup scans the
 * histograms, as in moe_dispatch_layout), then the scatter, which adds each
 * token's workgroup prefix to the ranks and writes expand_idx itself, so no
 * finalize launch sits between them.  The ranking launch, which is latency
 * bound, also reads the token rows x ahead (ordinary loads, x contiguous:
 * all rows up to 240 MB, else the first 128 MB) so that the scatter finds
 * them in the 256 MB Infinity Cache instead of interleaving row reads from
 * HBM with its writes.  When every row was read ahead, the bf16 scatter
 * runs with fewer waves in flight (at most 7 workgroups of 64 threads per
 * compute unit), which narrows the window of destination rows being
 * written at once.
 *
 *  x, x_stride, bs, hidden                   as for moe_dispatch.
 *  expert_ids, k, num_experts, align         as for moe_dispatch_layout.
 *  expert_counts, ep_send_counts, expand_idx out, as for moe_dispatch_layout.
 *  expand_x, expand_x_stride, capacity_rows, out_dtype, quant_scales
 *                                            as for moe_dispatch.
 *  status         out int32 [1] or NULL: MOE_FLAG_ID_RANGE | MOE_FLAG_DUP_ID |
 *                     MOE_FLAG_GUARD of this call, overwritten.
 *  workspace      as for moe_dispatch_layout (unused, may be NULL, when the
 *                     single launch applies).
 */
int moe_dispatch_fused(const void* x, int64_t x_stride, int32_t bs, int32_t hidden,
                       const int32_t* expert_ids, int32_t k, int32_t num_experts, int32_t align,
                       int32_t* expert_counts, int32_t* ep_send_counts, int32_t* expand_idx,
                       void* expand_x, int64_t expand_x_stride, int64_t capacity_rows,
                       int32_t out_dtype, float* quant_scales, int32_t* status, void* workspace,
                       size_t workspace_bytes, void* stream);

/*
 * moe_dispatch_fused without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  It allocates nothing; the layout's
 * workspace is a static device array of moe_noalloc_scratch_bytes() bytes
 * (5 MiB) that each GPU the library runs on holds until the process ends,
 * its address looked up once per device on the first call there.  Every
 * batch of at most 2^20 pairs fits (more with fewer experts: the rule is
 * moe_dispatch_layout_workspace_size(bs, k, num_experts) <=
 * moe_noalloc_scratch_bytes()); a larger one returns MOE_ERR_SCRATCH and
 * enqueues nothing.  All calls on one GPU share its array: calls that
 * overlap on one GPU (from other streams or threads) race and must be
 * serialised by the caller.  Arguments, outputs and results are those of
 * moe_dispatch_fused, bit for bit.
 */
int moe_dispatch_fused_noalloc(const void* x, int64_t x_stride, int32_t bs, int32_t hidden,
                               const int32_t* expert_ids, int32_t k, int32_t num_experts,
                               int32_t align, int32_t* expert_counts, int32_t* ep_send_counts,
                               int32_t* expand_idx, void* expand_x, int64_t expand_x_stride,
                               int64_t capacity_rows, int32_t out_dtype, float* quant_scales,
                               int32_t* status, void* stream);

/* Bytes of the static per-GPU scratch moe_dispatch_fused_noalloc uses. */
size_t moe_noalloc_scratch_bytes(void);

/*
 * Combine: gather each token's K expert-output rows back and form
 *   x_out[t,:] = sum_j expert_scales[t,j] * expand_x[slot(t,j), :] + shared_expert_x[t,:]
 * (the formula of the npu_moe_distribute_combine page, with the shared expert
 * added without a weight as its expert_scales parameter note states).
 *
 * Arithmetic: fp32, a fused multiply-add chain over j = 0..k-1 in order,
 * starting from +0; then the shared row is added; then one round to nearest
 * even into bf16.  Pairs with expand_idx < 0 or an out-of-range id contribute
 * nothing.
 *
 *  expand_x       in  bf16 expert outputs [capacity_rows, hidden], row stride
 *                     expand_x_stride; 16-byte aligned, stride*2 % 16 == 0.
 *  expert_ids, expand_idx, ep_send_counts
 *                 in  the same layout outputs the dispatch used.
 *  expert_scales  in  fp32 [bs, k] row-major, contiguous.
 *  shared_expert_x in bf16 [bs, hidden], row stride shared_stride, or NULL.
 *  bs, hidden     in  as for moe_dispatch (bs*hidden/8 < 2^31).
 *  x_out          out bf16 [bs, hidden], contiguous (the page requires a
 *                     contiguous output), 16-byte aligned.
 *  status         in/out int32 [1] or NULL: MOE_FLAG_GUARD is OR-ed in when a
 *                     pair's row lies at or beyond capacity_rows; that pair
 *                     contributes nothing to its token's sum.
 */
int moe_combine(const void* expand_x, int64_t expand_x_stride, int64_t capacity_rows,
                const int32_t* expert_ids, const int32_t* expand_idx,
                const int32_t* ep_send_counts, const float* expert_scales,
                const void* shared_expert_x, int64_t shared_stride, int32_t bs, int32_t hidden,
                int32_t k, int32_t num_experts, void* x_out, int32_t* status, void* stream);

/*
 * Quantised-transfer combine: the same weighted gather-sum as moe_combine,
 * with the expert outputs in the e4m3 format that moe_dispatch emits (the
 * combine page's comm_quant_mode names a quantised transfer on this path;
 * its dtype is unreadable there, and this library reads it as that format).
 *
 *   x_out[t,h] = bf16( fma-chain_j( expert_scales[t,j],
 *                         e4m3(expand_x[slot(t,j), h]) * quant_scales[slot(t,j), h/128] )
 *                      + shared_expert_x[t,h] )
 *
 * Each term is dequantised with one fp32 multiply before the fused
 * multiply-add chain over j ascending from +0; then the shared row is added
 * and the sum rounded to nearest even into bf16.
 *
 *  expand_x       in  e4m3fn codes [capacity_rows, hidden], row stride
 *                     expand_x_stride bytes (>= hidden, multiple of 16),
 *                     16-byte aligned.
 *  quant_scales   in  fp32 [capacity_rows, hidden/128] row-major.
 *  hidden         in  a multiple of 128, <= 65536, bs*hidden/8 < 2^31.
 *  other arguments as for moe_combine.
 */
int moe_combine_fp8(const void* expand_x, int64_t expand_x_stride, int64_t capacity_rows,
                    const float* quant_scales, const int32_t* expert_ids,
                    const int32_t* expand_idx, const int32_t* ep_send_counts,
                    const float* expert_scales, const void* shared_expert_x,
                    int64_t shared_stride, int32_t bs, int32_t hidden, int32_t k,
                    int32_t num_experts, void* x_out, int32_t* status, void* stream);

/*
 * The replica-aware layout and the dispatch over replicas in one call: the
 * results of moe_dispatch_layout_replicated followed by moe_dispatch with
 * expert_ids = replica_ids and num_experts = num_replicas, on the same
 * stream, bit for bit (replica ids, counts, offsets, ranks, dispatched rows,
 * padding rows left unwritten, e4m3 codes and scales, status bits).  As in
 * moe_dispatch_fused, batches of more than 2048 pairs take the ranking
 * launch, which also reads the token rows ahead into the Infinity Cache (x
 * contiguous; all rows up to 240 MB, else the first 128 MB), and the
 * scatter, which completes expand_idx; a bf16 scatter of rows that were all
 * read ahead runs with fewer waves in flight.  Batches of at most 2048
 * pairs take one layout launch and the scatter launch.
 *
 *  x, x_stride, hidden, expand_x, expand_x_stride, capacity_rows, out_dtype,
 *  quant_scales               as for moe_dispatch (over num_replicas).
 *  expert_ids, bs, k, num_experts, replica_offsets, replica_thresholds,
 *  num_replicas, seed, align, replica_ids, replica_counts, ep_send_counts,
 *  expand_idx, workspace      as for moe_dispatch_layout_replicated.
 *  status         out int32 [1] or NULL: MOE_FLAG_ID_RANGE | MOE_FLAG_DUP_ID |
 *                     MOE_FLAG_REPLICA | MOE_FLAG_GUARD of this call,
 *                     overwritten.
 * Returns the first error of the two calls' argument rules (nothing is
 * enqueued), MOE_ERR_WORKSPACE, MOE_ERR_HIP if a launch fails, else 0.
 */
int moe_dispatch_fused_replicated(const void* x, int64_t x_stride, int32_t bs, int32_t hidden,
                                  const int32_t* expert_ids, int32_t k, int32_t num_experts,
                                  const int32_t* replica_offsets,
                                  const uint32_t* replica_thresholds, int32_t num_replicas,
                                  uint64_t seed, int32_t align, int32_t* replica_ids,
                                  int32_t* replica_counts, int32_t* ep_send_counts,
                                  int32_t* expand_idx, void* expand_x, int64_t expand_x_stride,
                                  int64_t capacity_rows, int32_t out_dtype, float* quant_scales,
                                  int32_t* status, void* workspace, size_t workspace_bytes,
                                  void* stream);

/*
 * Compensation planner (host code, host pointers; no GPU involved).  The
 * DeepEP compensation PR (Python section) describes a water-filling
 * chunk-migration planner with expert-affinity batching, a makespan guard, a
 * cost-aware no-op and 128-aligned chunks; the TEMPO summary (section 2)
 * prices an expert on a device as an activation floor plus a cost per
 * 128-row M-tile.  With expert e homed on rank e / (E / ep_world_size), the
 * load of a rank is the sum over the experts it computes of
 *   activation_cost + tile_cost * ceil(rows / 128).
 * The planner repeatedly moves whole 128-row chunks of one expert from the
 * most to the least loaded rank (lowest index on ties): the move minimising
 * the pair's new maximum, ties to an expert the receiver already computes,
 * then the lower expert id, then fewer chunks; a move is admitted only if
 * the receiver stays below the current makespan; it stops when the two loads
 * differ by at most one tile, no move is admitted or max_moves are made, and
 * returns no move at all if the makespan fell by less than min_gain.
 *
 *  expert_counts   in  int32 [num_experts] (host): tokens per expert, >= 0,
 *                      e.g. the layout's expert_counts summed over ranks.
 *  ep_world_size   in  >= 1, dividing num_experts (<= 2^20).
 *  tile_cost, activation_cost, min_gain
 *                  in  integer cost units (tile_cost > 0, others >= 0).
 *  moves           out int32 [max_moves][4] (host): expert, source rank,
 *                      destination rank, rows (a multiple of 128).
 *  n_moves         out number of moves written.
 *  rank_loads      out int64 [ep_world_size] (host): loads after the plan.
 *  makespan_before, makespan_after, ideal
 *                  out (nullable): largest load before and after, and the
 *                      ideal bound ceil(sum of starting loads / ranks).
 * Returns MOE_ERR_INVALID_ARG for bad arguments; never touches the GPU.
 */
int moe_plan_compensation(const int32_t* expert_counts, int32_t num_experts,
                          int32_t ep_world_size, int64_t tile_cost, int64_t activation_cost,
                          int64_t min_gain, int32_t max_moves, int32_t* moves, int32_t* n_moves,
                          int64_t* rank_loads, int64_t* makespan_before, int64_t* makespan_after,
                          int64_t* ideal);

#ifdef __cplusplus
}
#endif

#endif /* MOE_DISPATCH_H */
