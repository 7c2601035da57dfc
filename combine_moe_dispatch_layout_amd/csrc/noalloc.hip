// noalloc.hip -- moe_dispatch_fused without a caller workspace, for callers
// that cannot allocate (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).  The multi-workgroup layout's workspace
// (ranking workgroups' histograms and flags, the arrival counter and the
// ranks within each workgroup) lives in `scratch`, a static device array
// that every GPU the library runs on holds until the process ends.
//
// Host code never passes `scratch` itself: its name there is a host-side
// stand-in, not a device address.  The address on each device is looked up
// once, with that device current, and kept per device.
//
// Initial contents: only the arrival counter must start at zero.  Static
// device memory is zero-filled when the code object is loaded, and every
// call returns the counter to zero (the last ranking workgroup resets it),
// so each call finds it at zero; the rest of the scratch is written before
// it is read within a call.  Every call on one GPU shares its array, so
// calls that overlap on one GPU (other streams or threads) race and must
// be serialised by the caller.
#include <mutex>

#include "moe_internal.h"

namespace {

constexpr size_t kScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device

// The device the call's kernels run on: the stream's, or the current one
// for the null stream.
hipError_t stream_device(hipStream_t stream, int* device) {
  if (stream == nullptr) return hipGetDevice(device);
  return hipStreamGetDevice(stream, device);
}

// Device address of `scratch` on `device`, looked up on first use with that
// device current (the caller's current device is restored).
int scratch_on(int device, void** out) {
  if (device < 0 || device >= kMaxDevices) return MOE_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[device] == nullptr) {
    int current = -1;
    if (hipGetDevice(&current) != hipSuccess) return MOE_ERR_HIP;
    if (current != device && hipSetDevice(device) != hipSuccess) return MOE_ERR_HIP;
    void* p = nullptr;
    const hipError_t err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (current != device && hipSetDevice(current) != hipSuccess) return MOE_ERR_HIP;
    if (err != hipSuccess || p == nullptr) return MOE_ERR_HIP;
    g_scratch_ptr[device] = p;
  }
  *out = g_scratch_ptr[device];
  return MOE_OK;
}

}  // namespace

extern "C" {

size_t moe_noalloc_scratch_bytes(void) { return kScratchBytes; }

int moe_dispatch_fused_noalloc(const void* x, int64_t x_stride, int32_t bs, int32_t hidden,
                               const int32_t* expert_ids, int32_t k, int32_t num_experts,
                               int32_t align, int32_t* expert_counts, int32_t* ep_send_counts,
                               int32_t* expand_idx, void* expand_x, int64_t expand_x_stride,
                               int64_t capacity_rows, int32_t out_dtype, float* quant_scales,
                               int32_t* status, void* stream) {
  // Invalid layout arguments report 0 bytes here and are refused by the
  // fused call below with its own code.
  const size_t need = moe_dispatch_layout_workspace_size(bs, k, num_experts);
  if (need > kScratchBytes) return MOE_ERR_SCRATCH;
  void* ws = nullptr;
  if (need > 0) {
    int device = -1;
    if (stream_device(static_cast<hipStream_t>(stream), &device) != hipSuccess)
      return MOE_ERR_HIP;
    const int rc = scratch_on(device, &ws);
    if (rc != MOE_OK) return rc;
  }
  return moe_dispatch_fused(x, x_stride, bs, hidden, expert_ids, k, num_experts, align,
                            expert_counts, ep_send_counts, expand_idx, expand_x,
                            expand_x_stride, capacity_rows, out_dtype, quant_scales, status, ws,
                            need > 0 ? kScratchBytes : 0, stream);
}

}  // extern "C"
