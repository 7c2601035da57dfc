/*
 * moe_probe.h -- measurement probe exported by libmoe_dispatch.so beside the
 * MoE path's C ABI (moe_dispatch.h).  It is not a step of the path: it gives
 * the practical bandwidth ceiling of plain streaming kernels that move bytes
 * in the same read : write mix as the dispatch (1 : K) and the combine
 * ((K + 1) : 1), so that a kernel's achieved GB/s can be read against both
 * the 8 TB/s HBM peak and what a plain kernel of that shape reaches.
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

#ifdef __cplusplus
}
#endif

#endif /* MOE_PROBE_H */
