/*
 * moe_probe.h -- measurement support exported by libmoe_dispatch.so beside
 * the MoE path's C ABI (moe_dispatch.h).  None of it is a step of the path:
 *  - moe_probe_stream_mix gives the practical bandwidth ceiling of plain
 *    streaming kernels that move bytes in the same read : write mix as the
 *    dispatch (1 : K) and the combine ((K + 1) : 1), so that a kernel's
 *    achieved GB/s can be read against both the 8 TB/s HBM peak and what a
 *    plain kernel of that shape reaches;
 *  - moe_time_next_launches binds HIP events to the library's next kernel
 *    launches, so each kernel is timed by its own start and end rather than
 *    by events recorded around it.
 * Conventions (device pointers, stream as void*, status codes) are those of
 * moe_dispatch.h.
 */
#ifndef MOE_PROBE_H
#define MOE_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * For each item i in [0, items): read `reads` rows of row_bytes from src and
 * write their XOR to `writes` rows of dst, in 16-byte vectors with
 * non-temporal loads and stores.
 *
 *  src, src_rows_total  in  device buffer of src_rows_total rows of row_bytes,
 *                           16-byte aligned.
 *  dst, dst_rows_total  out device buffer of dst_rows_total rows, 16-byte
 *                           aligned.
 *  items                in  >= 0.
 *  row_bytes            in  a positive multiple of 16, at most 2^20.
 *  reads, writes        in  1..16.
 *  src_rows             in  int32 [items * reads] source row of each read, or
 *                           NULL for row i*reads + r (which must then fit
 *                           src_rows_total).
 *  dst_rows             in  int32 [items * writes] destination row of each
 *                           write, or NULL for row i*writes + w (which must
 *                           then fit dst_rows_total).
 * Row indices outside a buffer are skipped.  Returns MOE_ERR_INVALID_ARG
 * (1) for bad arguments (nothing is enqueued), MOE_ERR_HIP (4) if the launch
 * fails, else 0.
 */
int moe_probe_stream_mix(const void* src, int64_t src_rows_total, void* dst,
                         int64_t dst_rows_total, int32_t items, int32_t row_bytes, int32_t reads,
                         int32_t writes, const int32_t* src_rows, const int32_t* dst_rows,
                         void* stream);

/*
 * Binds the next n kernel launches that the calling host thread makes
 * through this library (by any entry point, in launch order) to n event
 * pairs.  Launch i is enqueued with hipExtLaunchKernel, which stamps
 * start_events[i] and stop_events[i] (hipEvent_t passed as void*, created
 * by the caller with timing enabled and owned by it) with the kernel's own
 * start and end, so hipEventElapsedTime(start_events[i], stop_events[i]) is
 * that kernel's execution time.  Events recorded on the stream around a
 * kernel also hold the gap before it starts; these do not.
 *
 * An entry point makes one launch per kernel: moe_dispatch_layout one or two
 * (one when a single workgroup ranks the batch); moe_dispatch one, or two (a
 * read-ahead of the token rows, then the scatter) for bf16 output from
 * contiguous rows of 32 to 240 MB; moe_dispatch_fused one (fused kernel, bs*k <= 2048) or two (the
 * layout's ranking launch, then the scatter); moe_combine and
 * moe_combine_fp8 one.  Calls that return an error or have nothing to do
 * launch nothing and leave the pairs bound.
 *
 *  n   in  0..16; a new call replaces the pairs still bound, and n = 0 only
 *          drops them.
 * Bindings are per host thread and meant for eager launches; bind no pairs
 * while the stream is being captured.  Returns
 * MOE_ERR_INVALID_ARG (1) for n outside 0..16 or a NULL event among the
 * first n pairs (the bound pairs are then unchanged), else 0.
 */
int moe_time_next_launches(void* const* start_events, void* const* stop_events, int32_t n);

/* Number of pairs bound by moe_time_next_launches that no launch has taken
 * yet, on the calling host thread. */
int32_t moe_time_unused_launches(void);

/*
 * An empty kernel of `workgroups` workgroups of 128 threads: the fixed cost
 * of one launch of that grid (workgroup dispatch and the end-of-kernel
 * release, no memory traffic), the latency floor against which the
 * decode-sized kernels are read.
 *  workgroups  in  >= 1.
 * Returns MOE_ERR_INVALID_ARG (1) for workgroups < 1, MOE_ERR_HIP (4) if the
 * launch fails, else 0.
 */
int moe_probe_empty(int32_t workgroups, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_PROBE_H */
