"""MI355X (gfx950) MoE token dispatch / combine.

A thin Python binding over ``libmoe_dispatch.so`` (C ABI in
``include/moe_dispatch.h``).  Every step of the path runs in the library's HIP
kernels; this module only marshals torch tensors (device memory and the
current stream) into pointers.  If the library is not built the import of the
entry points fails loudly -- there is no fallback.

Entry points (same names as the C ABI):

* ``moe_dispatch_layout(expert_ids, num_experts, align=128)`` ->
  ``Layout(expert_counts, ep_send_counts, expand_idx, status)``
* ``moe_dispatch(x, expert_ids, layout_or_arrays..., out_dtype="bf16")`` ->
  ``expand_x`` (and ``quant_scales`` for e4m3)
* ``moe_dispatch_fused(x, expert_ids, num_experts, align=128)`` ->
  ``(Layout, expand_x)`` (and ``quant_scales`` for e4m3): layout + dispatch in
  one call, one kernel launch for batches of at most 2048 pairs
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
"""

from __future__ import annotations

import ctypes
import os

import numpy as np
from typing import NamedTuple, Optional

import torch

__all__ = [
    "MoeError", "Layout", "library_path", "load_library",
    "moe_dispatch_capacity", "moe_dispatch_layout_workspace_size",
    "moe_dispatch_layout", "moe_dispatch_layout_ep", "moe_dispatch_layout_replicated",
    "moe_dispatch", "moe_dispatch_fused", "moe_dispatch_fused_replicated", "moe_combine",
    "moe_plan_compensation",
    "moe_combine_fp8", "moe_probe_stream_mix", "moe_time_next_launches",
    "moe_time_unused_launches",
    "MOE_BF16", "MOE_FP8_E4M3", "MOE_FLAG_ID_RANGE", "MOE_FLAG_DUP_ID", "MOE_FLAG_GUARD",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmoe_dispatch.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_WORKSPACE, MOE_ERR_UNSUPPORTED, MOE_ERR_HIP = range(5)
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
        "moe_combine": (ctypes.c_int, [P, i64, i64, P, P, P, P, P, i64, i32, i32, i32, i32, P,
                                       P, P]),
        "moe_combine_fp8": (ctypes.c_int, [P, i64, i64, P, P, P, P, P, P, i64, i32, i32, i32,
                                           i32, P, P, P]),
        "moe_plan_compensation": (ctypes.c_int, [P, i32, i32, i64, i64, i64, i32, P, P, P, P, P,
                                                 P]),
        "moe_dispatch_layout_ep": (ctypes.c_int, [P, i32, i32, i32, i32, i32, P, P, P, P, P, P,
                                                  sz, P]),
        "moe_probe_stream_mix": (ctypes.c_int, [P, i64, P, i64, i32, i32, i32, i32, P, P, P]),
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


# The current stream's raw handle.  torch's raw getter skips building a
# Stream object (about 0.1 us against 1.9 us per call, which matters for
# decode-sized steps); the public API serves where it is absent.
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(t: torch.Tensor) -> Optional[int]:
    if _raw_stream is not None:
        return _raw_stream(t.device.index)
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, dtype: torch.dtype, name: str, contiguous: bool = True) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _row_stride(t: torch.Tensor, name: str) -> int:
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be 2-D with unit column stride")
    return t.stride(0)


class Layout(NamedTuple):
    expert_counts: torch.Tensor   # int32 [E]
    ep_send_counts: torch.Tensor  # int32 [E+1], exclusive padded prefix, last = M_pad
    expand_idx: torch.Tensor      # int32 [BS*K], within-expert rank (-1 = dropped pair)
    status: torch.Tensor          # int32 [1], moe_flag bits


def moe_dispatch_capacity(bs: int, k: int, num_experts: int, align: int = 128) -> int:
    cap = load_library().moe_dispatch_capacity(bs, k, num_experts, align)
    if cap < 0:
        raise MoeError(MOE_ERR_INVALID_ARG, "invalid layout arguments")
    return int(cap)


def moe_dispatch_layout_workspace_size(bs: int, k: int, num_experts: int) -> int:
    return int(load_library().moe_dispatch_layout_workspace_size(bs, k, num_experts))


def moe_dispatch_layout(expert_ids: torch.Tensor, num_experts: int, align: int = 128, *,
                        out: Optional[Layout] = None,
                        workspace: Optional[torch.Tensor] = None) -> Layout:
    """Counts, padded prefix and stable ranks of a [BS, K] int32 routing."""
    _need(expert_ids, torch.int32, "expert_ids")
    if expert_ids.dim() != 2:
        raise ValueError("expert_ids must be [BS, K]")
    bs, k = expert_ids.shape
    dev = expert_ids.device
    if out is None:
        out = Layout(torch.empty(num_experts, dtype=torch.int32, device=dev),
                     torch.empty(num_experts + 1, dtype=torch.int32, device=dev),
                     torch.empty(bs * k, dtype=torch.int32, device=dev),
                     torch.empty(1, dtype=torch.int32, device=dev))
    ws_bytes = moe_dispatch_layout_workspace_size(bs, k, num_experts)
    if ws_bytes and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    rc = load_library().moe_dispatch_layout(
        _ptr(expert_ids), bs, k, num_experts, align, _ptr(out.expert_counts),
        _ptr(out.ep_send_counts), _ptr(out.expand_idx), _ptr(out.status), _ptr(workspace),
        0 if workspace is None else workspace.numel() * workspace.element_size(),
        _stream(expert_ids))
    _check(rc)
    return out


def moe_dispatch(x: torch.Tensor, expert_ids: torch.Tensor, expand_idx: torch.Tensor,
                 ep_send_counts: torch.Tensor, num_experts: int, *,
                 capacity_rows: Optional[int] = None, out_dtype: str = "bf16",
                 expand_x: Optional[torch.Tensor] = None,
                 quant_scales: Optional[torch.Tensor] = None,
                 status: Optional[torch.Tensor] = None, align: int = 128):
    """Scatter x [BS, H] bf16 into expand_x [capacity_rows, H] (bf16, or e4m3
    codes as uint8 plus fp32 scales [capacity_rows, H/128]).  Returns
    ``expand_x`` or ``(expand_x, quant_scales)``."""
    _need(x, torch.bfloat16, "x", contiguous=False)
    _need(expert_ids, torch.int32, "expert_ids")
    _need(expand_idx, torch.int32, "expand_idx")
    _need(ep_send_counts, torch.int32, "ep_send_counts")
    bs, hidden = x.shape
    k = expert_ids.shape[1]
    dtype = {"bf16": MOE_BF16, "fp8": MOE_FP8_E4M3, "e4m3": MOE_FP8_E4M3}[out_dtype]
    if capacity_rows is None:
        capacity_rows = (expand_x.shape[0] if expand_x is not None
                         else moe_dispatch_capacity(bs, k, num_experts, align))
    if expand_x is None:
        expand_x = torch.empty((capacity_rows, hidden),
                               dtype=torch.bfloat16 if dtype == MOE_BF16 else torch.uint8,
                               device=x.device)
    if dtype == MOE_FP8_E4M3 and quant_scales is None:
        quant_scales = torch.empty((capacity_rows, hidden // 128), dtype=torch.float32,
                                   device=x.device)
    rc = load_library().moe_dispatch(
        _ptr(x), _row_stride(x, "x"), bs, hidden, _ptr(expert_ids), _ptr(expand_idx),
        _ptr(ep_send_counts), k, num_experts, _ptr(expand_x), _row_stride(expand_x, "expand_x"),
        capacity_rows, dtype, _ptr(quant_scales) if dtype == MOE_FP8_E4M3 else None,
        _ptr(status), _stream(x))
    _check(rc)
    return expand_x if dtype == MOE_BF16 else (expand_x, quant_scales)


def moe_dispatch_fused(x: torch.Tensor, expert_ids: torch.Tensor, num_experts: int,
                       align: int = 128, *, out: Optional[Layout] = None,
                       capacity_rows: Optional[int] = None, out_dtype: str = "bf16",
                       expand_x: Optional[torch.Tensor] = None,
                       quant_scales: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None):
    """moe_dispatch_layout + moe_dispatch in one call (one launch for batches
    of at most 2048 pairs).  Returns ``(layout, expand_x)`` or
    ``(layout, expand_x, quant_scales)``."""
    _need(x, torch.bfloat16, "x", contiguous=False)
    _need(expert_ids, torch.int32, "expert_ids")
    if expert_ids.dim() != 2 or expert_ids.shape[0] != x.shape[0]:
        raise ValueError("expert_ids must be [BS, K] with BS = x.shape[0]")
    bs, hidden = x.shape
    k = expert_ids.shape[1]
    dev = x.device
    dtype = {"bf16": MOE_BF16, "fp8": MOE_FP8_E4M3, "e4m3": MOE_FP8_E4M3}[out_dtype]
    if out is None:
        out = Layout(torch.empty(num_experts, dtype=torch.int32, device=dev),
                     torch.empty(num_experts + 1, dtype=torch.int32, device=dev),
                     torch.empty(bs * k, dtype=torch.int32, device=dev),
                     torch.empty(1, dtype=torch.int32, device=dev))
    if capacity_rows is None:
        capacity_rows = (expand_x.shape[0] if expand_x is not None
                         else moe_dispatch_capacity(bs, k, num_experts, align))
    if expand_x is None:
        expand_x = torch.empty((capacity_rows, hidden),
                               dtype=torch.bfloat16 if dtype == MOE_BF16 else torch.uint8,
                               device=dev)
    if dtype == MOE_FP8_E4M3 and quant_scales is None:
        quant_scales = torch.empty((capacity_rows, hidden // 128), dtype=torch.float32,
                                   device=dev)
    ws_bytes = moe_dispatch_layout_workspace_size(bs, k, num_experts)
    if ws_bytes and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    rc = load_library().moe_dispatch_fused(
        _ptr(x), _row_stride(x, "x"), bs, hidden, _ptr(expert_ids), k, num_experts, align,
        _ptr(out.expert_counts), _ptr(out.ep_send_counts), _ptr(out.expand_idx),
        _ptr(expand_x), _row_stride(expand_x, "expand_x"), capacity_rows, dtype,
        _ptr(quant_scales) if dtype == MOE_FP8_E4M3 else None, _ptr(out.status),
        _ptr(workspace), 0 if workspace is None else workspace.numel() * workspace.element_size(),
        _stream(x))
    _check(rc)
    return (out, expand_x) if dtype == MOE_BF16 else (out, expand_x, quant_scales)


def moe_combine(expand_x: torch.Tensor, expert_ids: torch.Tensor, expand_idx: torch.Tensor,
                ep_send_counts: torch.Tensor, expert_scales: torch.Tensor,
                shared_expert_x: Optional[torch.Tensor], num_experts: int, *,
                out: Optional[torch.Tensor] = None,
                status: Optional[torch.Tensor] = None) -> torch.Tensor:
    """x_out[t] = sum_j expert_scales[t,j] * expand_x[slot(t,j)] + shared_expert_x[t]."""
    _need(expand_x, torch.bfloat16, "expand_x", contiguous=False)
    _need(expert_ids, torch.int32, "expert_ids")
    _need(expand_idx, torch.int32, "expand_idx")
    _need(ep_send_counts, torch.int32, "ep_send_counts")
    _need(expert_scales, torch.float32, "expert_scales")
    bs, k = expert_ids.shape
    cap, hidden = expand_x.shape
    shared_stride = 0
    if shared_expert_x is not None:
        _need(shared_expert_x, torch.bfloat16, "shared_expert_x", contiguous=False)
        shared_stride = _row_stride(shared_expert_x, "shared_expert_x")
    if out is None:
        out = torch.empty((bs, hidden), dtype=torch.bfloat16, device=expand_x.device)
    _need(out, torch.bfloat16, "out")
    rc = load_library().moe_combine(
        _ptr(expand_x), _row_stride(expand_x, "expand_x"), cap, _ptr(expert_ids),
        _ptr(expand_idx), _ptr(ep_send_counts), _ptr(expert_scales), _ptr(shared_expert_x),
        shared_stride, bs, hidden, k, num_experts, _ptr(out), _ptr(status), _stream(expand_x))
    _check(rc)
    return out


def moe_combine_fp8(expand_x: torch.Tensor, quant_scales: torch.Tensor, expert_ids: torch.Tensor,
                    expand_idx: torch.Tensor, ep_send_counts: torch.Tensor,
                    expert_scales: torch.Tensor, shared_expert_x: Optional[torch.Tensor],
                    num_experts: int, *, out: Optional[torch.Tensor] = None,
                    status: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Combine over e4m3 expert rows (uint8 codes [cap, H]) with fp32 scales
    [cap, H/128], each term dequantised before the weighted sum."""
    _need(expand_x, torch.uint8, "expand_x", contiguous=False)
    _need(quant_scales, torch.float32, "quant_scales")
    _need(expert_ids, torch.int32, "expert_ids")
    _need(expand_idx, torch.int32, "expand_idx")
    _need(ep_send_counts, torch.int32, "ep_send_counts")
    _need(expert_scales, torch.float32, "expert_scales")
    bs, k = expert_ids.shape
    cap, hidden = expand_x.shape
    if quant_scales.shape != (cap, hidden // 128):
        raise ValueError("quant_scales must be [capacity_rows, hidden/128]")
    shared_stride = 0
    if shared_expert_x is not None:
        _need(shared_expert_x, torch.bfloat16, "shared_expert_x", contiguous=False)
        shared_stride = _row_stride(shared_expert_x, "shared_expert_x")
    if out is None:
        out = torch.empty((bs, hidden), dtype=torch.bfloat16, device=expand_x.device)
    _need(out, torch.bfloat16, "out")
    rc = load_library().moe_combine_fp8(
        _ptr(expand_x), _row_stride(expand_x, "expand_x"), cap, _ptr(quant_scales),
        _ptr(expert_ids), _ptr(expand_idx), _ptr(ep_send_counts), _ptr(expert_scales),
        _ptr(shared_expert_x), shared_stride, bs, hidden, k, num_experts, _ptr(out),
        _ptr(status), _stream(expand_x))
    _check(rc)
    return out


def moe_dispatch_layout_replicated(expert_ids: torch.Tensor, num_experts: int,
                                   replica_offsets: torch.Tensor,
                                   replica_thresholds: torch.Tensor, seed: int,
                                   align: int = 128, *, out: Optional[Layout] = None,
                                   replica_ids: Optional[torch.Tensor] = None,
                                   workspace: Optional[torch.Tensor] = None):
    """Choose a physical replica per pair (SplitMix64 draw against cumulative
    uint32 thresholds, given as int32 or uint32 bit patterns) and lay the
    pairs out over the replicas.  Returns ``(replica_ids [BS, K], Layout)``."""
    _need(expert_ids, torch.int32, "expert_ids")
    _need(replica_offsets, torch.int32, "replica_offsets")
    if replica_thresholds.dtype not in (torch.int32, torch.uint32):
        raise ValueError("replica_thresholds must hold uint32 bit patterns (int32 or uint32)")
    _need(replica_thresholds, replica_thresholds.dtype, "replica_thresholds")
    bs, k = expert_ids.shape
    p = replica_thresholds.numel()
    dev = expert_ids.device
    if out is None:
        out = Layout(torch.empty(p, dtype=torch.int32, device=dev),
                     torch.empty(p + 1, dtype=torch.int32, device=dev),
                     torch.empty(bs * k, dtype=torch.int32, device=dev),
                     torch.empty(1, dtype=torch.int32, device=dev))
    if replica_ids is None:
        replica_ids = torch.empty((bs, k), dtype=torch.int32, device=dev)
    ws_bytes = moe_dispatch_layout_workspace_size(bs, k, p)
    if ws_bytes and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    rc = load_library().moe_dispatch_layout_replicated(
        _ptr(expert_ids), bs, k, num_experts, _ptr(replica_offsets), _ptr(replica_thresholds), p,
        seed & 0xFFFFFFFFFFFFFFFF, align, _ptr(replica_ids), _ptr(out.expert_counts),
        _ptr(out.ep_send_counts), _ptr(out.expand_idx), _ptr(out.status), _ptr(workspace),
        0 if workspace is None else workspace.numel() * workspace.element_size(),
        _stream(expert_ids))
    _check(rc)
    return replica_ids, out


def moe_dispatch_fused_replicated(x: torch.Tensor, expert_ids: torch.Tensor, num_experts: int,
                                  replica_offsets: torch.Tensor,
                                  replica_thresholds: torch.Tensor, seed: int,
                                  align: int = 128, *, out: Optional[Layout] = None,
                                  replica_ids: Optional[torch.Tensor] = None,
                                  capacity_rows: Optional[int] = None, out_dtype: str = "bf16",
                                  expand_x: Optional[torch.Tensor] = None,
                                  quant_scales: Optional[torch.Tensor] = None,
                                  workspace: Optional[torch.Tensor] = None):
    """moe_dispatch_layout_replicated + moe_dispatch over the replicas in one
    call.  Returns ``(replica_ids, layout, expand_x)`` or ``(replica_ids,
    layout, expand_x, quant_scales)``."""
    _need(x, torch.bfloat16, "x", contiguous=False)
    _need(expert_ids, torch.int32, "expert_ids")
    _need(replica_offsets, torch.int32, "replica_offsets")
    if replica_thresholds.dtype not in (torch.int32, torch.uint32):
        raise ValueError("replica_thresholds must hold uint32 bit patterns (int32 or uint32)")
    _need(replica_thresholds, replica_thresholds.dtype, "replica_thresholds")
    if expert_ids.dim() != 2 or expert_ids.shape[0] != x.shape[0]:
        raise ValueError("expert_ids must be [BS, K] with BS = x.shape[0]")
    bs, hidden = x.shape
    k = expert_ids.shape[1]
    p = replica_thresholds.numel()
    dev = x.device
    dtype = {"bf16": MOE_BF16, "fp8": MOE_FP8_E4M3, "e4m3": MOE_FP8_E4M3}[out_dtype]
    if out is None:
        out = Layout(torch.empty(p, dtype=torch.int32, device=dev),
                     torch.empty(p + 1, dtype=torch.int32, device=dev),
                     torch.empty(bs * k, dtype=torch.int32, device=dev),
                     torch.empty(1, dtype=torch.int32, device=dev))
    if replica_ids is None:
        replica_ids = torch.empty((bs, k), dtype=torch.int32, device=dev)
    if capacity_rows is None:
        capacity_rows = (expand_x.shape[0] if expand_x is not None
                         else moe_dispatch_capacity(bs, k, p, align))
    if expand_x is None:
        expand_x = torch.empty((capacity_rows, hidden),
                               dtype=torch.bfloat16 if dtype == MOE_BF16 else torch.uint8,
                               device=dev)
    if dtype == MOE_FP8_E4M3 and quant_scales is None:
        quant_scales = torch.empty((capacity_rows, hidden // 128), dtype=torch.float32,
                                   device=dev)
    ws_bytes = moe_dispatch_layout_workspace_size(bs, k, p)
    if ws_bytes and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    rc = load_library().moe_dispatch_fused_replicated(
        _ptr(x), _row_stride(x, "x"), bs, hidden, _ptr(expert_ids), k, num_experts,
        _ptr(replica_offsets), _ptr(replica_thresholds), p, seed & 0xFFFFFFFFFFFFFFFF, align,
        _ptr(replica_ids), _ptr(out.expert_counts), _ptr(out.ep_send_counts),
        _ptr(out.expand_idx), _ptr(expand_x), _row_stride(expand_x, "expand_x"), capacity_rows,
        dtype, _ptr(quant_scales) if dtype == MOE_FP8_E4M3 else None, _ptr(out.status),
        _ptr(workspace), 0 if workspace is None else workspace.numel() * workspace.element_size(),
        _stream(x))
    _check(rc)
    if dtype == MOE_BF16:
        return replica_ids, out, expand_x
    return replica_ids, out, expand_x, quant_scales


def moe_dispatch_layout_ep(expert_ids: torch.Tensor, num_experts: int, ep_world_size: int,
                           align: int = 128, *, out: Optional[Layout] = None,
                           rank_offsets: Optional[torch.Tensor] = None,
                           workspace: Optional[torch.Tensor] = None):
    """The layout plus per-destination-rank send offsets (experts split evenly
    and contiguously over ``ep_world_size`` ranks).  Returns
    ``(Layout, rank_offsets int32 [ws+1])``."""
    _need(expert_ids, torch.int32, "expert_ids")
    bs, k = expert_ids.shape
    dev = expert_ids.device
    if out is None:
        out = Layout(torch.empty(num_experts, dtype=torch.int32, device=dev),
                     torch.empty(num_experts + 1, dtype=torch.int32, device=dev),
                     torch.empty(bs * k, dtype=torch.int32, device=dev),
                     torch.empty(1, dtype=torch.int32, device=dev))
    if rank_offsets is None:
        rank_offsets = torch.empty(max(ep_world_size, 0) + 1, dtype=torch.int32, device=dev)
    ws_bytes = moe_dispatch_layout_workspace_size(bs, k, num_experts)
    if ws_bytes and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    rc = load_library().moe_dispatch_layout_ep(
        _ptr(expert_ids), bs, k, num_experts, ep_world_size, align, _ptr(out.expert_counts),
        _ptr(out.ep_send_counts), _ptr(rank_offsets), _ptr(out.expand_idx), _ptr(out.status),
        _ptr(workspace), 0 if workspace is None else workspace.numel() * workspace.element_size(),
        _stream(expert_ids))
    _check(rc)
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
        if not t.is_cuda or t.dim() != 2 or not t.is_contiguous():
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
