// probe.hip -- a streaming probe with the byte mixes of the dispatch and the
// combine, for the practical-ceiling figures reported beside the 8 TB/s HBM
// peak.  It is measurement support, not a step of the MoE path.
//
// Item i reads R rows and writes W rows of row_bytes each, in 16-byte
// vectors with non-temporal loads and stores, one workgroup of 128 threads
// per (item, 128-vector chunk) as in the dispatch and combine kernels, with
// the item's row indices fetched once by lanes 0..R+W-1:
//   read r  comes from row src_rows[i*R + r]  (i*R + r when src_rows is NULL)
//   write w goes to   row dst_rows[i*W + w]  (i*W + w when dst_rows is NULL)
// Every written vector is the XOR of the R vectors read, so every read is
// consumed.  R = 1, W = K has the dispatch's 1 : K mix; R = K + 1, W = 1 the
// combine's (K expert rows + the shared row) : 1 mix.  With the row arrays a
// random permutation reproduces the scattered side of the real layout
// without its metadata.  Row indices outside the buffers are skipped.
#include "moe_internal.h"
#include "moe_probe.h"

namespace moe {
namespace {

constexpr int kProbeThreads = 128;
constexpr int kProbeMaxRows = 16;

// Row of slot j of the item: reads first (j < R), then writes.  Lanes
// 0..R+W-1 fetch them once and every wave broadcasts them with readlane, so
// no load or store waits on an index fetched just before it.
__device__ __forceinline__ int64_t probe_row(int j, int64_t item, int32_t R, int32_t W,
                                             const int32_t* src_rows, const int32_t* dst_rows) {
  if (j < R) return src_rows ? (int64_t)src_rows[item * R + j] : item * R + j;
  const int w = j - R;
  return dst_rows ? (int64_t)dst_rows[item * W + w] : item * W + w;
}

__device__ __forceinline__ int64_t broadcast64(int64_t x, int lane) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int32_t)(x & 0xFFFFFFFF), lane);
  const int32_t hi = __builtin_amdgcn_readlane((int32_t)(x >> 32), lane);
  return (int64_t)(((uint64_t)(uint32_t)hi << 32) | lo);
}

// R_T / W_T > 0: compile-time counts; 0: the runtime counts R / W (up to 16).
template <int R_T, int W_T>
__global__ __launch_bounds__(kProbeThreads) void stream_mix_kernel(
    const u32x4* __restrict__ src, int64_t src_total, u32x4* __restrict__ dst, int64_t dst_total,
    int32_t nvec, int32_t nchunks, int32_t R_rt, int32_t W_rt,
    const int32_t* __restrict__ src_rows, const int32_t* __restrict__ dst_rows) {
  constexpr int RM = R_T > 0 ? R_T : kProbeMaxRows;
  constexpr int WM = W_T > 0 ? W_T : kProbeMaxRows;
  const int32_t R = R_T > 0 ? R_T : R_rt;
  const int32_t W = W_T > 0 ? W_T : W_rt;
  const int64_t item = blockIdx.x / nchunks;
  const int32_t chunk = blockIdx.x - (int32_t)(item * nchunks);
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t mine = (lane < R + W) ? probe_row(lane, item, R, W, src_rows, dst_rows) : -1;
  int64_t rrow[RM], wrow[WM];
#pragma unroll
  for (int r = 0; r < RM; ++r) rrow[r] = broadcast64(mine, r);
#pragma unroll
  for (int w = 0; w < WM; ++w) wrow[w] = broadcast64(mine, R + w < kWave ? R + w : 0);

  const int32_t v = chunk * kProbeThreads + threadIdx.x;
  if (v >= nvec) return;  // no barrier follows
  u32x4 acc = {0u, 0u, 0u, 0u};
  u32x4 val[RM];
#pragma unroll
  for (int r = 0; r < RM; ++r) {
    val[r] = u32x4{0u, 0u, 0u, 0u};
    if (r < R && rrow[r] >= 0 && rrow[r] < src_total)
      val[r] = load_stream(src + rrow[r] * nvec + v);
  }
#pragma unroll
  for (int r = 0; r < RM; ++r) acc ^= val[r];
#pragma unroll
  for (int w = 0; w < WM; ++w)
    if (w < W && wrow[w] >= 0 && wrow[w] < dst_total) store_stream(acc, dst + wrow[w] * nvec + v);
}

// Does nothing: the fixed cost of a launch (dispatch of the workgroups, the
// end-of-kernel release) with no memory traffic, the latency floor of a
// kernel of that grid.
__global__ __launch_bounds__(kProbeThreads) void empty_kernel() {}

}  // namespace
}  // namespace moe

extern "C" int moe_probe_empty(int32_t workgroups, void* stream) {
  if (workgroups < 1) return MOE_ERR_INVALID_ARG;
  moe::launch_kernel(moe::empty_kernel, dim3((uint32_t)workgroups), moe::kProbeThreads,
                     static_cast<hipStream_t>(stream));
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

extern "C" int moe_probe_stream_mix(const void* src, int64_t src_rows_total, void* dst,
                                    int64_t dst_rows_total, int32_t items, int32_t row_bytes,
                                    int32_t reads, int32_t writes, const int32_t* src_rows,
                                    const int32_t* dst_rows, void* stream) {
  if (items < 0 || row_bytes <= 0 || row_bytes % 16 != 0 || row_bytes > (1 << 20))
    return MOE_ERR_INVALID_ARG;
  if (reads < 1 || reads > moe::kProbeMaxRows || writes < 1 || writes > moe::kProbeMaxRows)
    return MOE_ERR_INVALID_ARG;
  if (src_rows_total < 0 || dst_rows_total < 0) return MOE_ERR_INVALID_ARG;
  if (items == 0) return MOE_OK;
  if (src == nullptr || dst == nullptr) return MOE_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15u)
    return MOE_ERR_INVALID_ARG;
  if (src_rows == nullptr && (int64_t)items * reads > src_rows_total) return MOE_ERR_INVALID_ARG;
  if (dst_rows == nullptr && (int64_t)items * writes > dst_rows_total) return MOE_ERR_INVALID_ARG;
  const int32_t nvec = row_bytes / 16;
  const int32_t nchunks = (nvec + moe::kProbeThreads - 1) / moe::kProbeThreads;
  // the grid's thread count must fit 32 bits
  if ((int64_t)items * nchunks * moe::kProbeThreads > (int64_t)UINT32_MAX)
    return MOE_ERR_INVALID_ARG;
  const dim3 grid((uint32_t)(items * nchunks));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const moe::u32x4* sv = static_cast<const moe::u32x4*>(src);
  moe::u32x4* dv = static_cast<moe::u32x4*>(dst);
#define MOE_PROBE(RT, WT)                                                                 \
  moe::launch_kernel(moe::stream_mix_kernel<RT, WT>, grid, moe::kProbeThreads, s,         \
      sv, src_rows_total, dv, dst_rows_total, nvec, nchunks, reads, writes, src_rows, dst_rows)
  // Compile-time counts for the dispatch (1 : K) and combine (K + 1 : 1) mixes.
  if (reads == 1 && writes == 2) MOE_PROBE(1, 2);
  else if (reads == 1 && writes == 4) MOE_PROBE(1, 4);
  else if (reads == 1 && writes == 8) MOE_PROBE(1, 8);
  else if (reads == 1 && writes == 16) MOE_PROBE(1, 16);
  else if (reads == 3 && writes == 1) MOE_PROBE(3, 1);
  else if (reads == 5 && writes == 1) MOE_PROBE(5, 1);
  else if (reads == 9 && writes == 1) MOE_PROBE(9, 1);
  else MOE_PROBE(0, 0);
#undef MOE_PROBE
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}
