"""MI355X (gfx950) MoE token dispatch / combine.

A thin Python binding over ``libmoe_dispatch.so`` (C ABI in
``include/moe_dispatch.h``).  Every step of the path runs in the library's HIP
kernels; this module only marshals torch tensors (device memory and the
current stream) into pointers.  If the library is not built the import of the
entry points fails loudly -- there is no fallback.

Before a call reaches the library, every tensor it passes is checked against
the call's sizes (device, dtype, contiguity, rows and columns, lengths), so
a mismatch raises ValueError instead of reaching the GPU.  The routing and
scatter calls take ``check=True`` to wait for the GPU and raise
MoeStatusError when the status word reports dropped pairs (a row beyond
capacity_rows, an out-of-range id, a replica table without a replica) or
repeated ids; it is off by default because it synchronises.

Entry points (same names as the C ABI):

* ``moe_dispatch_layout(expert_ids, num_experts, align=128)`` ->
  ``Layout(expert_counts, ep_send_counts, expand_idx, status)``
* ``moe_dispatch(x, expert_ids, layout_or_arrays..., out_dtype="bf16")`` ->
  ``expand_x`` (and ``quant_scales`` for e4m3)
* ``moe_dispatch_fused(x, expert_ids, num_experts, align=128)`` ->
  ``(Layout, expand_x)`` (and ``quant_scales`` for e4m3): layout + dispatch in
  one call, one kernel launch for batches of at most 2048 pairs, two above
* ``moe_combine(expand_x, expert_ids, expand_idx, ep_send_counts,
  expert_scales, shared_expert_x)`` -> ``x_out``
* ``moe_combine_fp8(expand_x_codes, quant_scales, ...)`` -> ``x_out`` (expert
  rows in the e4m3 + per-128-channel scale format, dequantised in the gather)
* ``moe_dispatch_layout_ep(expert_ids, num_experts, ep_world_size)`` ->
  ``(Layout, rank_offsets [ws+1])``
* ``moe_dispatch_layout_replicated(expert_ids, num_experts, replica_offsets,
  replica_thresholds, seed)`` -> ``(replica_ids, Layout over replicas)``
* ``moe_dispatch_fused_replicated(x, expert_ids, num_experts, replica_offsets,
  replica_thresholds, seed)`` -> ``(replica_ids, Layout, expand_x[,
  quant_scales])`` (the replica-aware layout and the dispatch in one call)
* ``moe_plan_compensation(expert_counts, ep_world_size, tile_cost,
  activation_cost)`` -> dict (host-side 128-aligned chunk-migration plan)
* ``moe_dispatch_capacity`` / ``moe_dispatch_layout_workspace_size``
* ``moe_probe_stream_mix`` (measurement only: a plain streaming kernel with a
  chosen read : write row mix, for practical-ceiling figures)
* ``moe_time_next_launches(pairs)`` / ``moe_time_unused_launches()``
  (measurement only: torch events stamped with the next kernels' own start
  and end)
* ``prepare(entry, *args, **kwargs)`` -> ``Prepared``: an entry point's call
  checked once, for loops that repeat it on the same tensors (a call then
  only launches)
"""

from __future__ import annotations

import ctypes
import os
import threading

import numpy as np
from typing import NamedTuple, Optional

import torch

__all__ = [
    "MoeError", "MoeStatusError", "Layout", "library_path", "load_library",
    "moe_dispatch_capacity", "moe_dispatch_layout_workspace_size",
    "moe_dispatch_layout", "moe_dispatch_layout_ep", "moe_dispatch_layout_replicated",
    "moe_dispatch", "moe_dispatch_fused", "moe_dispatch_fused_replicated", "moe_combine",
    "moe_dispatch_fused_noalloc", "moe_noalloc_scratch_bytes",
    "moe_plan_compensation",
    "moe_combine_fp8", "moe_probe_stream_mix", "moe_probe_empty", "moe_time_next_launches",
    "moe_time_unused_launches", "prepare", "Prepared",
    "MOE_BF16", "MOE_FP8_E4M3", "MOE_FLAG_ID_RANGE", "MOE_FLAG_DUP_ID", "MOE_FLAG_GUARD",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmoe_dispatch.so")

(MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_WORKSPACE, MOE_ERR_UNSUPPORTED, MOE_ERR_HIP,
 MOE_ERR_SCRATCH) = range(6)
MOE_BF16, MOE_FP8_E4M3 = 0, 1
MOE_FLAG_ID_RANGE, MOE_FLAG_DUP_ID, MOE_FLAG_GUARD, MOE_FLAG_REPLICA = 1, 2, 4, 8

_lib = None


class MoeError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{msg} (status {code})")
        self.code = code


def library_path() -> str:
    return _LIB_PATH


def load_library() -> ctypes.CDLL:
    """Load the HIP library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"{_LIB_PATH} is missing: build it with "
            "`python -m combine_moe_dispatch_layout_amd.build` (no CPU fallback exists)")
    lib = ctypes.CDLL(_LIB_PATH)
    P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    sigs = {
        "moe_abi_version": (ctypes.c_int, []),
        "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "moe_dispatch_capacity": (i64, [i32, i32, i32, i32]),
        "moe_dispatch_layout_workspace_size": (sz, [i32, i32, i32]),
        "moe_dispatch_layout": (ctypes.c_int, [P, i32, i32, i32, i32, P, P, P, P, P, sz, P]),
        "moe_dispatch": (ctypes.c_int, [P, i64, i32, i32, P, P, P, i32, i32, P, i64, i64, i32,
                                        P, P, P]),
        "moe_dispatch_fused": (ctypes.c_int, [P, i64, i32, i32, P, i32, i32, i32, P, P, P, P,
                                              i64, i64, i32, P, P, P, sz, P]),
        "moe_dispatch_fused_noalloc": (ctypes.c_int, [P, i64, i32, i32, P, i32, i32, i32, P,
                                                      P, P, P, i64, i64, i32, P, P, P]),
        "moe_noalloc_scratch_bytes": (sz, []),
        "moe_combine": (ctypes.c_int, [P, i64, i64, P, P, P, P, P, i64, i32, i32, i32, i32, P,
                                       P, P]),
        "moe_combine_fp8": (ctypes.c_int, [P, i64, i64, P, P, P, P, P, P, i64, i32, i32, i32,
                                           i32, P, P, P]),
        "moe_plan_compensation": (ctypes.c_int, [P, i32, i32, i64, i64, i64, i32, P, P, P, P, P,
                                                 P]),
        "moe_dispatch_layout_ep": (ctypes.c_int, [P, i32, i32, i32, i32, i32, P, P, P, P, P, P,
                                                  sz, P]),
        "moe_probe_stream_mix": (ctypes.c_int, [P, i64, P, i64, i32, i32, i32, i32, P, P, P]),
        "moe_probe_empty": (ctypes.c_int, [i32, P]),
        "moe_time_next_launches": (ctypes.c_int, [P, P, i32]),
        "moe_time_unused_launches": (i32, []),
        "moe_dispatch_layout_replicated": (ctypes.c_int, [P, i32, i32, i32, P, P, i32,
                                                          ctypes.c_uint64, i32, P, P, P, P, P, P,
                                                          sz, P]),
        "moe_dispatch_fused_replicated": (ctypes.c_int, [P, i64, i32, i32, P, i32, i32, P, P,
                                                         i32, ctypes.c_uint64, i32, P, P, P, P,
                                                         P, i64, i64, i32, P, P, P, sz, P]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(rc: int) -> None:
    if rc != MOE_OK:
        raise MoeError(rc, load_library().moe_status_string(rc).decode())


# While prepare() runs an entry point, its library launch is recorded here
# (per host thread) instead of being made.
_recording = threading.local()


def _launch(fn, *args) -> int:
    calls = getattr(_recording, "calls", None)
    if calls is not None:
        calls.append((fn, args))
        return MOE_OK
    return fn(*args)


class Prepared:
    """A library call validated once: calling it repeats the same launch
    (same tensors, same stream) with no argument checks, for tight serving
    loops launched from the host.  ``result`` holds what the entry point
    returned (its output tensors, which every call overwrites)."""

    def __init__(self, name: str, fn, args, result):
        self.name = name
        self.result = result
        self._fn = fn
        self._args = args

    def __call__(self):
        rc = self._fn(*self._args)
        if rc != MOE_OK:
            _check(rc)
        return self.result


def prepare(entry, *args, **kwargs) -> Prepared:
    """Run entry point ``entry`` (e.g. ``moe_dispatch_fused``) with these
    arguments through all of its checks and output allocation, but instead of
    launching, return a Prepared call that launches it.  The tensors it was
    given or allocated must stay alive and keep their shapes, strides and
    devices; their contents may change between calls.  The launch goes to
    the stream that was current when prepare() ran.  ``check=True`` cannot
    be prepared (it synchronises)."""
    if kwargs.get("check"):
        raise ValueError("check=True cannot be prepared")
    _recording.calls = []
    try:
        result = entry(*args, **kwargs)
        calls = _recording.calls
    finally:
        _recording.calls = None
    if len(calls) != 1:
        raise ValueError(f"{getattr(entry, '__name__', entry)} does not make one library launch")
    fn, raw = calls[0]
    # Arguments converted once to the C types the function declares, so a
    # call skips the per-argument conversion.
    types = getattr(fn, "argtypes", None)
    conv = raw if types is None else tuple(
        a if a is None or isinstance(a, t) else t(a) for t, a in zip(types, raw))
    return Prepared(getattr(entry, "__name__", str(entry)), fn, conv, result)


class MoeStatusError(MoeError):
    """Raised by calls made with ``check=True`` when the device-side status
    word reports pairs that were dropped or malformed routing."""

    def __init__(self, flags: int, call: str):
        names = [n for bit, n in ((MOE_FLAG_ID_RANGE, "ID_RANGE"), (MOE_FLAG_DUP_ID, "DUP_ID"),
                                  (MOE_FLAG_GUARD, "GUARD"), (MOE_FLAG_REPLICA, "REPLICA"))
                 if flags & bit]
        super().__init__(flags, f"{call}: status flags {'|'.join(names)}")
        self.flags = flags


def _raise_on_status(status: torch.Tensor, call: str) -> None:
    """check=True: wait for the call (a host synchronisation) and raise on
    any status bit: out-of-range ids, repeated ids in a row, a slot beyond
    capacity_rows (its pair was dropped) or a replica table without a
    replica for some draw."""
    flags = int(status.reshape(-1)[0].item())
    if flags:
        raise MoeStatusError(flags, call)


# The current stream's raw handle.  torch's raw getter skips building a
# Stream object (about 0.1 us against 1.9 us per call, which matters for
# decode-sized steps); the public API serves where it is absent.
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)

# Device type every tensor argument must have.  The argument checks below
# run before any library call; the CPU test tier sets this to "cpu" (with the
# library stubbed out) to exercise them without a GPU.
_DEVICE_TYPE = "cuda"


def _stream(t: torch.Tensor) -> Optional[int]:
    if _raw_stream is not None:
        return _raw_stream(t.get_device())
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _nbytes(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else t.numel() * t.element_size()


# The checks read each tensor's facts once through torch's cheapest
# accessors (get_device() rather than .device): a decode-sized step is
# bound by host time, and these run on every call.

def _device_of(t, name: str) -> int:
    """The device index of a tensor argument (-1 on the CPU test tier)."""
    try:
        dev = t.get_device()
    except AttributeError:
        raise ValueError(f"{name} must be a tensor") from None
    if (dev >= 0) != (_DEVICE_TYPE == "cuda"):
        raise ValueError(f"{name} must be a device tensor")
    return dev


def _need(t, dtype, name: str, contiguous: bool = True, device: Optional[int] = None) -> int:
    """t is a tensor of `dtype` (a dtype or a tuple of them) on the library's
    device type (on device index `device` when given), contiguous unless told
    not.  Returns its device index."""
    try:
        dev = t.get_device()
        dt = t.dtype
    except AttributeError:
        raise ValueError(f"{name} must be a tensor") from None
    if (dev >= 0) != (_DEVICE_TYPE == "cuda"):
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and dev != device:
        raise ValueError(f"{name} is on device {dev}, the call's tensors on {device}")
    if dt is not dtype and (not isinstance(dtype, tuple) or dt not in dtype):
        want = " or ".join(map(str, dtype)) if isinstance(dtype, tuple) else str(dtype)
        raise ValueError(f"{name} must be {want}, got {dt}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return dev


def _need_len(t: torch.Tensor, n: int, name: str) -> None:
    """A contiguous array the kernels index up to element n - 1."""
    if t.numel() < n:
        raise ValueError(f"{name} holds {t.numel()} elements, the call needs {n}")


def _row_stride(t: torch.Tensor, name: str) -> int:
    st = t.stride()
    if len(st) != 2 or st[1] != 1:
        raise ValueError(f"{name} must be 2-D with unit column stride")
    return st[0]


def _need_rows(t: torch.Tensor, rows: int, cols: int, name: str) -> int:
    """A 2-D row buffer with at least `rows` rows of exactly `cols` columns
    and unit column stride; returns its row stride."""
    st = t.stride()
    if len(st) != 2 or st[1] != 1:
        raise ValueError(f"{name} must be 2-D with unit column stride")
    shape = t.shape
    if shape[1] != cols:
        raise ValueError(f"{name} rows hold {shape[1]} columns, the call needs {cols}")
    if shape[0] < rows:
        raise ValueError(f"{name} has {shape[0]} rows, the call needs {rows}")
    return st[0]


def _need_ids(expert_ids, name: str = "expert_ids", bs: Optional[int] = None,
              device: Optional[int] = None):
    _need(expert_ids, torch.int32, name, device=device)
    shape = expert_ids.shape
    if len(shape) != 2:
        raise ValueError(f"{name} must be [BS, K]")
    if bs is not None and shape[0] != bs:
        raise ValueError(f"{name} has {shape[0]} rows, x has {bs}")
    return shape


def _dtype_code(out_dtype: str) -> int:
    codes = {"bf16": MOE_BF16, "fp8": MOE_FP8_E4M3, "e4m3": MOE_FP8_E4M3}
    if out_dtype not in codes:
        raise ValueError(f"out_dtype must be one of {sorted(codes)}, got {out_dtype!r}")
    return codes[out_dtype]


def _new(shape, dtype, device: int):
    return torch.empty(shape, dtype=dtype, device=torch.device(_DEVICE_TYPE, device)
                       if device >= 0 else "cpu")


class Layout(NamedTuple):
    expert_counts: torch.Tensor   # int32 [E]
    ep_send_counts: torch.Tensor  # int32 [E+1], exclusive padded prefix, last = M_pad
    expand_idx: torch.Tensor      # int32 [BS*K], within-expert rank (-1 = dropped pair)
    status: torch.Tensor          # int32 [1], moe_flag bits


_LAYOUT_NAMES = ("out.expert_counts", "out.ep_send_counts", "out.expand_idx", "out.status")


def _layout(out: Optional[Layout], n_experts: int, n_pairs: int, device: int) -> Layout:
    """The caller's Layout, checked against the call's sizes, or a new one."""
    if out is None:
        return Layout(_new(n_experts, torch.int32, device),
                      _new(n_experts + 1, torch.int32, device),
                      _new(n_pairs, torch.int32, device), _new(1, torch.int32, device))
    for t, n, name in zip(out, (n_experts, n_experts + 1, n_pairs, 1), _LAYOUT_NAMES):
        _need(t, torch.int32, name, device=device)
        if t.numel() < n:
            raise ValueError(f"{name} holds {t.numel()} elements, the call needs {n}")
    return out


def _workspace(workspace: Optional[torch.Tensor], bs: int, k: int, n_experts: int, device):
    """The caller's workspace (checked for size), or a new zero-filled one;
    None when the layout needs none."""
    ws_bytes = moe_dispatch_layout_workspace_size(bs, k, n_experts)
    if workspace is None:
        return _new(ws_bytes, torch.uint8, device).zero_() if ws_bytes else None
    _need(workspace, workspace.dtype, "workspace", device=device)
    if _nbytes(workspace) < ws_bytes:
        raise ValueError(f"workspace holds {_nbytes(workspace)} bytes, the call needs {ws_bytes}")
    return workspace


def _scatter_outputs(expand_x, quant_scales, capacity_rows, bs, k, hidden, n_experts, align,
                     dtype, device):
    """The dispatched-row buffer (and e4m3 scales) of a scatter: the caller's,
    checked against capacity_rows and the row size, or new ones."""
    if capacity_rows is None:
        capacity_rows = (expand_x.shape[0] if expand_x is not None
                         else moe_dispatch_capacity(bs, k, n_experts, align))
    if capacity_rows < 0:
        raise ValueError("capacity_rows must be >= 0")
    row_dtype = torch.bfloat16 if dtype == MOE_BF16 else torch.uint8
    if expand_x is None:
        expand_x = _new((capacity_rows, hidden), row_dtype, device)
    _need(expand_x, row_dtype, "expand_x", contiguous=False, device=device)
    _need_rows(expand_x, capacity_rows, hidden, "expand_x")
    if dtype == MOE_FP8_E4M3:
        if hidden % 128:
            raise ValueError("e4m3 output needs hidden to be a multiple of 128")
        if quant_scales is None:
            quant_scales = _new((capacity_rows, hidden // 128), torch.float32, device)
        _need(quant_scales, torch.float32, "quant_scales", device=device)
        _need_rows(quant_scales, capacity_rows, hidden // 128, "quant_scales")
    return capacity_rows, expand_x, quant_scales


# Size queries, memoised per library (their answers depend only on the
# arguments): the checks ask for them on every call.
_sizes: dict = {}


def moe_dispatch_capacity(bs: int, k: int, num_experts: int, align: int = 128) -> int:
    lib = load_library()
    key = (id(lib), "cap", bs, k, num_experts, align)
    cap = _sizes.get(key)
    if cap is None:
        cap = _sizes.setdefault(key, int(lib.moe_dispatch_capacity(bs, k, num_experts, align)))
    if cap < 0:
        raise MoeError(MOE_ERR_INVALID_ARG, "invalid layout arguments")
    return cap


def moe_dispatch_layout_workspace_size(bs: int, k: int, num_experts: int) -> int:
    """Bytes of device workspace the layout needs (0: none).  A workspace must
    be zero-filled before its first use; every call leaves its first word (an
    arrival counter) zero, the only part that needs initial contents."""
    lib = load_library()
    key = (id(lib), "ws", bs, k, num_experts)
    n = _sizes.get(key)
    if n is None:
        n = _sizes.setdefault(key, int(lib.moe_dispatch_layout_workspace_size(bs, k,
                                                                             num_experts)))
    return n


def moe_dispatch_layout(expert_ids: torch.Tensor, num_experts: int, align: int = 128, *,
                        out: Optional[Layout] = None,
                        workspace: Optional[torch.Tensor] = None,
                        check: bool = False) -> Layout:
    """Counts, padded prefix and stable ranks of a [BS, K] int32 routing.
    With check=True the call waits for the GPU and raises MoeStatusError if
    the status word reports out-of-range or repeated ids."""
    bs, k = _need_ids(expert_ids)
    dev = expert_ids.get_device()
    out = _layout(out, num_experts, bs * k, dev)
    workspace = _workspace(workspace, bs, k, num_experts, dev)
    rc = _launch(load_library().moe_dispatch_layout,
        _ptr(expert_ids), bs, k, num_experts, align, _ptr(out.expert_counts),
        _ptr(out.ep_send_counts), _ptr(out.expand_idx), _ptr(out.status), _ptr(workspace),
        _nbytes(workspace), _stream(expert_ids))
    _check(rc)
    if check:
        _raise_on_status(out.status, "moe_dispatch_layout")
    return out


def _routes(expert_ids, expand_idx, ep_send_counts, num_experts, bs, dev):
    """The layout outputs a dispatch or combine reads, checked for size."""
    _, k = _need_ids(expert_ids, bs=bs, device=dev)
    _need(expand_idx, torch.int32, "expand_idx", device=dev)
    _need_len(expand_idx, bs * k, "expand_idx")
    _need(ep_send_counts, torch.int32, "ep_send_counts", device=dev)
    _need_len(ep_send_counts, num_experts + 1, "ep_send_counts")
    return k


def _status_word(status: Optional[torch.Tensor], check: bool, dev: int):
    """The in/out status word of a scatter or combine: the caller's (checked),
    or with check=True a new zeroed one."""
    if status is None:
        return _new(1, torch.int32, dev).zero_() if check else None
    _need(status, torch.int32, "status", device=dev)
    _need_len(status, 1, "status")
    return status


def moe_dispatch(x: torch.Tensor, expert_ids: torch.Tensor, expand_idx: torch.Tensor,
                 ep_send_counts: torch.Tensor, num_experts: int, *,
                 capacity_rows: Optional[int] = None, out_dtype: str = "bf16",
                 expand_x: Optional[torch.Tensor] = None,
                 quant_scales: Optional[torch.Tensor] = None,
                 status: Optional[torch.Tensor] = None, align: int = 128, check: bool = False):
    """Scatter x [BS, H] bf16 into expand_x [capacity_rows, H] (bf16, or e4m3
    codes as uint8 plus fp32 scales [capacity_rows, H/128]).  Returns
    ``expand_x`` or ``(expand_x, quant_scales)``.  A capacity_rows below
    moe_dispatch_capacity is allowed (a caller that knows the padded total
    may size the buffer to it); pairs past it are dropped and flagged
    MOE_FLAG_GUARD, which check=True turns into MoeStatusError."""
    dev = _need(x, torch.bfloat16, "x", contiguous=False)
    if x.dim() != 2:
        raise ValueError("x must be [BS, H]")
    bs, hidden = x.shape
    k = _routes(expert_ids, expand_idx, ep_send_counts, num_experts, bs, dev)
    dtype = _dtype_code(out_dtype)
    capacity_rows, expand_x, quant_scales = _scatter_outputs(
        expand_x, quant_scales, capacity_rows, bs, k, hidden, num_experts, align, dtype, dev)
    status = _status_word(status, check, dev)
    rc = _launch(load_library().moe_dispatch,
        _ptr(x), _row_stride(x, "x"), bs, hidden, _ptr(expert_ids), _ptr(expand_idx),
        _ptr(ep_send_counts), k, num_experts, _ptr(expand_x), _row_stride(expand_x, "expand_x"),
        capacity_rows, dtype, _ptr(quant_scales) if dtype == MOE_FP8_E4M3 else None,
        _ptr(status), _stream(x))
    _check(rc)
    if check:
        _raise_on_status(status, "moe_dispatch")
    return expand_x if dtype == MOE_BF16 else (expand_x, quant_scales)


def moe_dispatch_fused(x: torch.Tensor, expert_ids: torch.Tensor, num_experts: int,
                       align: int = 128, *, out: Optional[Layout] = None,
                       capacity_rows: Optional[int] = None, out_dtype: str = "bf16",
                       expand_x: Optional[torch.Tensor] = None,
                       quant_scales: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None, check: bool = False):
    """moe_dispatch_layout + moe_dispatch in one call (one launch for batches
    of at most 2048 pairs, two above).  Returns ``(layout, expand_x)`` or
    ``(layout, expand_x, quant_scales)``.  check=True waits for the GPU and
    raises MoeStatusError on any status bit."""
    dev = _need(x, torch.bfloat16, "x", contiguous=False)
    if x.dim() != 2:
        raise ValueError("x must be [BS, H]")
    bs, hidden = x.shape
    _, k = _need_ids(expert_ids, bs=bs, device=dev)
    dtype = _dtype_code(out_dtype)
    out = _layout(out, num_experts, bs * k, dev)
    capacity_rows, expand_x, quant_scales = _scatter_outputs(
        expand_x, quant_scales, capacity_rows, bs, k, hidden, num_experts, align, dtype, dev)
    workspace = _workspace(workspace, bs, k, num_experts, dev)
    rc = _launch(load_library().moe_dispatch_fused,
        _ptr(x), _row_stride(x, "x"), bs, hidden, _ptr(expert_ids), k, num_experts, align,
        _ptr(out.expert_counts), _ptr(out.ep_send_counts), _ptr(out.expand_idx),
        _ptr(expand_x), _row_stride(expand_x, "expand_x"), capacity_rows, dtype,
        _ptr(quant_scales) if dtype == MOE_FP8_E4M3 else None, _ptr(out.status),
        _ptr(workspace), _nbytes(workspace), _stream(x))
    _check(rc)
    if check:
        _raise_on_status(out.status, "moe_dispatch_fused")
    return (out, expand_x) if dtype == MOE_BF16 else (out, expand_x, quant_scales)


def moe_dispatch_fused_noalloc(x: torch.Tensor, expert_ids: torch.Tensor, num_experts: int,
                               align: int = 128, *, out: Optional[Layout] = None,
                               capacity_rows: Optional[int] = None, out_dtype: str = "bf16",
                               expand_x: Optional[torch.Tensor] = None,
                               quant_scales: Optional[torch.Tensor] = None,
                               check: bool = False):
    """moe_dispatch_fused with the layout's workspace in the library's static
    per-GPU scratch (no device allocation by the call; pass `out`,
    `expand_x` and, for e4m3, `quant_scales` to allocate nothing at all).
    Batches whose workspace exceeds moe_noalloc_scratch_bytes() raise
    MoeError (MOE_ERR_SCRATCH).  Calls that overlap on one GPU race."""
    dev = _need(x, torch.bfloat16, "x", contiguous=False)
    if x.dim() != 2:
        raise ValueError("x must be [BS, H]")
    bs, hidden = x.shape
    _, k = _need_ids(expert_ids, bs=bs, device=dev)
    dtype = _dtype_code(out_dtype)
    out = _layout(out, num_experts, bs * k, dev)
    capacity_rows, expand_x, quant_scales = _scatter_outputs(
        expand_x, quant_scales, capacity_rows, bs, k, hidden, num_experts, align, dtype, dev)
    rc = _launch(load_library().moe_dispatch_fused_noalloc,
        _ptr(x), _row_stride(x, "x"), bs, hidden, _ptr(expert_ids), k, num_experts, align,
        _ptr(out.expert_counts), _ptr(out.ep_send_counts), _ptr(out.expand_idx),
        _ptr(expand_x), _row_stride(expand_x, "expand_x"), capacity_rows, dtype,
        _ptr(quant_scales) if dtype == MOE_FP8_E4M3 else None, _ptr(out.status), _stream(x))
    _check(rc)
    if check:
        _raise_on_status(out.status, "moe_dispatch_fused_noalloc")
    return (out, expand_x) if dtype == MOE_BF16 else (out, expand_x, quant_scales)


def moe_noalloc_scratch_bytes() -> int:
    """Bytes of the static per-GPU scratch of moe_dispatch_fused_noalloc."""
    return int(load_library().moe_noalloc_scratch_bytes())


def _combine_rows(shared_expert_x, out, bs, hidden, dev):
    shared_stride = 0
    if shared_expert_x is not None:
        _need(shared_expert_x, torch.bfloat16, "shared_expert_x", contiguous=False, device=dev)
        shared_stride = _need_rows(shared_expert_x, bs, hidden, "shared_expert_x")
        if shared_expert_x.shape[0] != bs:
            raise ValueError(f"shared_expert_x has {shared_expert_x.shape[0]} rows, BS is {bs}")
    if out is None:
        out = _new((bs, hidden), torch.bfloat16, dev)
    _need(out, torch.bfloat16, "out", device=dev)
    if tuple(out.shape) != (bs, hidden):
        raise ValueError(f"out must be [{bs}, {hidden}], got {list(out.shape)}")
    return shared_stride, out


def moe_combine(expand_x: torch.Tensor, expert_ids: torch.Tensor, expand_idx: torch.Tensor,
                ep_send_counts: torch.Tensor, expert_scales: torch.Tensor,
                shared_expert_x: Optional[torch.Tensor], num_experts: int, *,
                out: Optional[torch.Tensor] = None,
                status: Optional[torch.Tensor] = None, check: bool = False) -> torch.Tensor:
    """x_out[t] = sum_j expert_scales[t,j] * expand_x[slot(t,j)] + shared_expert_x[t].
    check=True waits for the GPU and raises MoeStatusError if a slot fell
    outside expand_x (that pair contributed nothing)."""
    dev = _need(expand_x, torch.bfloat16, "expand_x", contiguous=False)
    bs, k = _need_ids(expert_ids, device=dev)
    _routes(expert_ids, expand_idx, ep_send_counts, num_experts, bs, dev)
    _need(expert_scales, torch.float32, "expert_scales", device=dev)
    _need_len(expert_scales, bs * k, "expert_scales")
    ys = _row_stride(expand_x, "expand_x")
    cap, hidden = expand_x.shape
    shared_stride, out = _combine_rows(shared_expert_x, out, bs, hidden, dev)
    status = _status_word(status, check, dev)
    rc = _launch(load_library().moe_combine,
        _ptr(expand_x), ys, cap, _ptr(expert_ids), _ptr(expand_idx), _ptr(ep_send_counts),
        _ptr(expert_scales), _ptr(shared_expert_x), shared_stride, bs, hidden, k, num_experts,
        _ptr(out), _ptr(status), _stream(expand_x))
    _check(rc)
    if check:
        _raise_on_status(status, "moe_combine")
    return out


def moe_combine_fp8(expand_x: torch.Tensor, quant_scales: torch.Tensor, expert_ids: torch.Tensor,
                    expand_idx: torch.Tensor, ep_send_counts: torch.Tensor,
                    expert_scales: torch.Tensor, shared_expert_x: Optional[torch.Tensor],
                    num_experts: int, *, out: Optional[torch.Tensor] = None,
                    status: Optional[torch.Tensor] = None, check: bool = False) -> torch.Tensor:
    """Combine over e4m3 expert rows (uint8 codes [cap, H]) with fp32 scales
    [cap, H/128], each term dequantised before the weighted sum."""
    dev = _need(expand_x, torch.uint8, "expand_x", contiguous=False)
    bs, k = _need_ids(expert_ids, device=dev)
    _routes(expert_ids, expand_idx, ep_send_counts, num_experts, bs, dev)
    _need(expert_scales, torch.float32, "expert_scales", device=dev)
    _need_len(expert_scales, bs * k, "expert_scales")
    ys = _row_stride(expand_x, "expand_x")
    cap, hidden = expand_x.shape
    if hidden % 128:
        raise ValueError("e4m3 rows need hidden to be a multiple of 128")
    _need(quant_scales, torch.float32, "quant_scales", device=dev)
    if tuple(quant_scales.shape) != (cap, hidden // 128):
        raise ValueError("quant_scales must be [capacity_rows, hidden/128]")
    shared_stride, out = _combine_rows(shared_expert_x, out, bs, hidden, dev)
    status = _status_word(status, check, dev)
    rc = _launch(load_library().moe_combine_fp8,
        _ptr(expand_x), ys, cap, _ptr(quant_scales), _ptr(expert_ids), _ptr(expand_idx),
        _ptr(ep_send_counts), _ptr(expert_scales), _ptr(shared_expert_x), shared_stride, bs,
        hidden, k, num_experts, _ptr(out), _ptr(status), _stream(expand_x))
    _check(rc)
    if check:
        _raise_on_status(status, "moe_combine_fp8")
    return out


def _replica_tables(replica_offsets, replica_thresholds, num_experts, dev):
    _need(replica_offsets, torch.int32, "replica_offsets", device=dev)
    _need_len(replica_offsets, num_experts + 1, "replica_offsets")
    _need(replica_thresholds, (torch.int32, torch.uint32), "replica_thresholds", device=dev)
    return replica_thresholds.numel()


def _replica_ids(replica_ids, bs, k, dev):
    if replica_ids is None:
        return _new((bs, k), torch.int32, dev)
    _need(replica_ids, torch.int32, "replica_ids", device=dev)
    _need_len(replica_ids, bs * k, "replica_ids")
    return replica_ids


def moe_dispatch_layout_replicated(expert_ids: torch.Tensor, num_experts: int,
                                   replica_offsets: torch.Tensor,
                                   replica_thresholds: torch.Tensor, seed: int,
                                   align: int = 128, *, out: Optional[Layout] = None,
                                   replica_ids: Optional[torch.Tensor] = None,
                                   workspace: Optional[torch.Tensor] = None,
                                   check: bool = False):
    """Choose a physical replica per pair (SplitMix64 draw against cumulative
    uint32 thresholds, given as int32 or uint32 bit patterns) and lay the
    pairs out over the replicas.  Returns ``(replica_ids [BS, K], Layout)``."""
    bs, k = _need_ids(expert_ids)
    dev = expert_ids.get_device()
    p = _replica_tables(replica_offsets, replica_thresholds, num_experts, dev)
    out = _layout(out, p, bs * k, dev)
    replica_ids = _replica_ids(replica_ids, bs, k, dev)
    workspace = _workspace(workspace, bs, k, p, dev)
    rc = _launch(load_library().moe_dispatch_layout_replicated,
        _ptr(expert_ids), bs, k, num_experts, _ptr(replica_offsets), _ptr(replica_thresholds), p,
        seed & 0xFFFFFFFFFFFFFFFF, align, _ptr(replica_ids), _ptr(out.expert_counts),
        _ptr(out.ep_send_counts), _ptr(out.expand_idx), _ptr(out.status), _ptr(workspace),
        _nbytes(workspace), _stream(expert_ids))
    _check(rc)
    if check:
        _raise_on_status(out.status, "moe_dispatch_layout_replicated")
    return replica_ids, out


def moe_dispatch_fused_replicated(x: torch.Tensor, expert_ids: torch.Tensor, num_experts: int,
                                  replica_offsets: torch.Tensor,
                                  replica_thresholds: torch.Tensor, seed: int,
                                  align: int = 128, *, out: Optional[Layout] = None,
                                  replica_ids: Optional[torch.Tensor] = None,
                                  capacity_rows: Optional[int] = None, out_dtype: str = "bf16",
                                  expand_x: Optional[torch.Tensor] = None,
                                  quant_scales: Optional[torch.Tensor] = None,
                                  workspace: Optional[torch.Tensor] = None,
                                  check: bool = False):
    """moe_dispatch_layout_replicated + moe_dispatch over the replicas in one
    call.  Returns ``(replica_ids, layout, expand_x)`` or ``(replica_ids,
    layout, expand_x, quant_scales)``."""
    dev = _need(x, torch.bfloat16, "x", contiguous=False)
    if x.dim() != 2:
        raise ValueError("x must be [BS, H]")
    bs, hidden = x.shape
    _, k = _need_ids(expert_ids, bs=bs, device=dev)
    p = _replica_tables(replica_offsets, replica_thresholds, num_experts, dev)
    dtype = _dtype_code(out_dtype)
    out = _layout(out, p, bs * k, dev)
    replica_ids = _replica_ids(replica_ids, bs, k, dev)
    capacity_rows, expand_x, quant_scales = _scatter_outputs(
        expand_x, quant_scales, capacity_rows, bs, k, hidden, p, align, dtype, dev)
    workspace = _workspace(workspace, bs, k, p, dev)
    rc = _launch(load_library().moe_dispatch_fused_replicated,
        _ptr(x), _row_stride(x, "x"), bs, hidden, _ptr(expert_ids), k, num_experts,
        _ptr(replica_offsets), _ptr(replica_thresholds), p, seed & 0xFFFFFFFFFFFFFFFF, align,
        _ptr(replica_ids), _ptr(out.expert_counts), _ptr(out.ep_send_counts),
        _ptr(out.expand_idx), _ptr(expand_x), _row_stride(expand_x, "expand_x"), capacity_rows,
        dtype, _ptr(quant_scales) if dtype == MOE_FP8_E4M3 else None, _ptr(out.status),
        _ptr(workspace), _nbytes(workspace), _stream(x))
    _check(rc)
    if check:
        _raise_on_status(out.status, "moe_dispatch_fused_replicated")
    if dtype == MOE_BF16:
        return replica_ids, out, expand_x
    return replica_ids, out, expand_x, quant_scales


def moe_dispatch_layout_ep(expert_ids: torch.Tensor, num_experts: int, ep_world_size: int,
                           align: int = 128, *, out: Optional[Layout] = None,
                           rank_offsets: Optional[torch.Tensor] = None,
                           workspace: Optional[torch.Tensor] = None, check: bool = False):
    """The layout plus per-destination-rank send offsets (experts split evenly
    and contiguously over ``ep_world_size`` ranks).  Returns
    ``(Layout, rank_offsets int32 [ws+1])``."""
    bs, k = _need_ids(expert_ids)
    dev = expert_ids.get_device()
    out = _layout(out, num_experts, bs * k, dev)
    if rank_offsets is None:
        rank_offsets = _new(max(ep_world_size, 0) + 1, torch.int32, dev)
    _need(rank_offsets, torch.int32, "rank_offsets", device=dev)
    _need_len(rank_offsets, max(ep_world_size, 0) + 1, "rank_offsets")
    workspace = _workspace(workspace, bs, k, num_experts, dev)
    rc = _launch(load_library().moe_dispatch_layout_ep,
        _ptr(expert_ids), bs, k, num_experts, ep_world_size, align, _ptr(out.expert_counts),
        _ptr(out.ep_send_counts), _ptr(rank_offsets), _ptr(out.expand_idx), _ptr(out.status),
        _ptr(workspace), _nbytes(workspace), _stream(expert_ids))
    _check(rc)
    if check:
        _raise_on_status(out.status, "moe_dispatch_layout_ep")
    return out, rank_offsets


def moe_plan_compensation(expert_counts, ep_world_size: int, tile_cost: int,
                          activation_cost: int, min_gain: int = 0, max_moves: int = 1024) -> dict:
    """Host-side 128-aligned compensation plan over per-expert token counts
    (any int sequence, numpy array or CPU tensor).  Returns dict(moves=[(expert,
    src, dst, rows)], loads=[...], before, after, ideal)."""
    if isinstance(expert_counts, torch.Tensor):
        expert_counts = expert_counts.detach().cpu().numpy()
    counts = np.ascontiguousarray(expert_counts, dtype=np.int32)
    moves = np.zeros((max(max_moves, 1), 4), dtype=np.int32)
    n = ctypes.c_int32(0)
    loads = np.zeros(max(ep_world_size, 1), dtype=np.int64)
    before, after, ideal = ctypes.c_int64(0), ctypes.c_int64(0), ctypes.c_int64(0)
    rc = load_library().moe_plan_compensation(
        counts.ctypes.data, counts.size, ep_world_size, tile_cost, activation_cost, min_gain,
        max_moves, moves.ctypes.data, ctypes.byref(n), loads.ctypes.data, ctypes.byref(before),
        ctypes.byref(after), ctypes.byref(ideal))
    _check(rc)
    return {"moves": [tuple(int(v) for v in row) for row in moves[:n.value]],
            "loads": [int(v) for v in loads[:ep_world_size]], "before": before.value,
            "after": after.value, "ideal": ideal.value}


def moe_probe_stream_mix(src: torch.Tensor, dst: torch.Tensor, items: int, reads: int,
                         writes: int, src_rows: Optional[torch.Tensor] = None,
                         dst_rows: Optional[torch.Tensor] = None) -> None:
    """Measurement probe (include/moe_probe.h): item i XORs `reads` rows of
    src into `writes` rows of dst.  src / dst are contiguous 2-D device
    tensors whose rows are the probe's rows; src_rows / dst_rows optional
    int32 row indices."""
    for t, name in ((src, "src"), (dst, "dst")):
        if t.device.type != _DEVICE_TYPE or t.dim() != 2 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 2-D device tensor")
    row_bytes = src.shape[1] * src.element_size()
    if dst.shape[1] * dst.element_size() != row_bytes:
        raise ValueError("src and dst rows differ in size")
    for t, name in ((src_rows, "src_rows"), (dst_rows, "dst_rows")):
        if t is not None:
            _need(t, torch.int32, name)
    rc = load_library().moe_probe_stream_mix(
        _ptr(src), src.shape[0], _ptr(dst), dst.shape[0], items, row_bytes, reads, writes,
        _ptr(src_rows), _ptr(dst_rows), _stream(src))
    _check(rc)


def moe_probe_empty(workgroups: int, device: Optional[int] = None) -> None:
    """Measurement probe (include/moe_probe.h): an empty kernel of
    `workgroups` workgroups on the current stream of `device` (the current
    device when None), the latency floor of one launch of that grid."""
    dev = torch.cuda.current_device() if device is None else device
    stream = _raw_stream(dev) if _raw_stream is not None else \
        torch.cuda.current_stream(dev).cuda_stream
    _check(load_library().moe_probe_empty(workgroups, stream))


def moe_time_next_launches(pairs) -> None:
    """Binds the next len(pairs) kernel launches of this host thread to
    (start, stop) torch.cuda.Event pairs created with enable_timing=True
    (include/moe_probe.h): each event pair gets its kernel's own start and
    end, and start.elapsed_time(stop) is that kernel's time.  An event must
    have been recorded once so that it exists.  An empty list drops the
    pairs still bound."""
    pairs = list(pairs)
    handles = []
    for start, stop in pairs:
        for ev in (start, stop):
            if not isinstance(ev, torch.cuda.Event) or not ev.cuda_event:
                raise ValueError("pairs must hold torch.cuda.Event objects recorded once")
        handles.append((start.cuda_event, stop.cuda_event))
    arr = (ctypes.c_void_p * max(len(pairs), 1))
    starts = arr(*[h[0] for h in handles])
    stops = arr(*[h[1] for h in handles])
    _check(load_library().moe_time_next_launches(starts, stops, len(pairs)))


def moe_time_unused_launches() -> int:
    """Number of event pairs bound by moe_time_next_launches that no launch
    has taken yet (this host thread)."""
    return int(load_library().moe_time_unused_launches())
