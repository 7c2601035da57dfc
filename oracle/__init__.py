"""CPU oracle for MoE dispatch layout, dispatch and combine.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product
package never imports it and shares no code with it: the arithmetic lives in
``moe_oracle.c`` (plain C loops, built with gcc, not hipcc); this module only
moves numpy arrays in and out of it through ctypes.

What each function computes, and the passage it follows, is stated in
``moe_oracle.c``.  In short (npu_moe_distribute_combine API page: function
description, formula, parameters expert_ids / expand_idx / ep_send_counts /
expert_scales / shared_expert_x; TEMPO summary section 1 for the 128-row tile):

* ``layout``      -- per-expert counts, 128-padded exclusive prefix (E+1
  entries), stable within-expert rank per (token, k) pair.
* ``dispatch_bf16`` / ``dispatch_fp8`` -- copy (or e4m3-quantise with one fp32
  scale amax/448 per 128 channels) token rows into slot
  ``ep_send_counts[e] + expand_idx``.
* ``combine``     -- fp32 fused-multiply-add chain over k ascending, plus the
  unweighted shared row, rounded to bf16 (nearest-even).
* ``combine_fp8`` -- the same sum over e4m3 expert rows, each term dequantised
  as ``e4m3_value * scale`` (one binary32 multiply) first.
* ``layout_ep``   -- the layout plus per-destination-rank send offsets for
  E/ws contiguous experts per rank (combine page, A3 ep_send_counts shape).
* ``layout_replicated`` -- each pair picks a physical replica of its expert
  by a SplitMix64 draw against cumulative thresholds (TEMPO summary, section
  2, system integration), then the layout runs over the replicas.

Parity status: every function is pinned by the ``not gpu`` tests (brute force,
closed forms, invariants, library codecs); none is "parity unpinned".
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

OK = 0
ERR_INVALID_ARG = 1
ERR_UNSUPPORTED = 3
FLAG_ID_RANGE = 1
FLAG_DUP_ID = 2
FLAG_GUARD = 4
FLAG_REPLICA = 8

# Sentinel the oracle's dispatch buffers are prefilled with, so that rows the
# method leaves unwritten (padding) stay recognisable.
SENTINEL_BF16 = 0x7FBF  # a NaN payload no conversion produces
SENTINEL_FP8 = 0x7F     # e4m3fn NaN code, never produced from finite input
SENTINEL_SCALE = -1.0   # scales are never negative


class OracleArgError(ValueError):
    """The oracle rejected the arguments (same rule set as the library)."""

    def __init__(self, code: int):
        super().__init__(f"oracle rejected arguments (code {code})")
        self.code = code


def build(force: bool = False) -> str:
    """Compile ``moe_oracle.c`` with gcc into ``liboracle.so``."""
    with _lock:
        stale = (not os.path.exists(_LIB)) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC)
        if force or stale:
            tmp = _LIB + f".tmp{os.getpid()}"
            cmd = ["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-Wall",
                   "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"]
            subprocess.run(cmd, check=True)
            os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    build()
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    i32, i64 = ctypes.c_int32, ctypes.c_int64
    sig = {
        "oracle_capacity": (i64, [i32, i32, i32, i32]),
        "oracle_check_layout_args": (ctypes.c_int, [i32, i32, i32, i32]),
        "oracle_check_row_args": (ctypes.c_int, [i32, i32]),
        "oracle_layout": (ctypes.c_int, [P, i32, i32, i32, i32, P, P, P, P]),
        "oracle_dispatch_bf16": (ctypes.c_int, [P, i64, i32, i32, P, P, P, i32, i32, P, i64, i64, P]),
        "oracle_quantize_row_e4m3": (None, [P, i32, P, P]),
        "oracle_dispatch_fp8": (ctypes.c_int, [P, i64, i32, i32, P, P, P, i32, i32, P, i64, i64,
                                               P, P, P, P]),
        "oracle_combine": (ctypes.c_int, [P, i64, i64, P, P, P, P, P, i64, i32, i32, i32, i32,
                                          P, P]),
        "oracle_combine_fp8": (ctypes.c_int, [P, i64, i64, P, P, P, P, P, P, i64, i32, i32,
                                              i32, i32, P, P]),
        "oracle_layout_ep": (ctypes.c_int, [P, i32, i32, i32, i32, i32, P, P, P, P, P]),
        "oracle_splitmix64": (ctypes.c_uint64, [ctypes.c_uint64, ctypes.c_uint64]),
        "oracle_layout_replicated": (ctypes.c_int, [P, i32, i32, i32, P, P, i32, ctypes.c_uint64,
                                                    i32, P, P, P, P, P]),
        "oracle_f32_to_bf16_array": (None, [P, i64, P]),
        "oracle_f32_to_e4m3_array": (None, [P, i64, P]),
        "oracle_e4m3_to_f32_array": (None, [P, i64, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"] or a.ndim == 0
    return a.ctypes.data


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.int32)


# --------------------------------------------------------------------------
# Argument rules
# --------------------------------------------------------------------------

def capacity(bs: int, k: int, num_experts: int, align: int = 128) -> int:
    """Rows that always hold the padded layout (worst case over routings)."""
    return int(_load().oracle_capacity(bs, k, num_experts, align))


def check_layout_args(bs: int, k: int, num_experts: int, align: int = 128) -> int:
    return int(_load().oracle_check_layout_args(bs, k, num_experts, align))


def check_row_args(hidden: int, dtype: int) -> int:
    return int(_load().oracle_check_row_args(hidden, dtype))


# --------------------------------------------------------------------------
# Codecs (array forms)
# --------------------------------------------------------------------------

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    _load().oracle_f32_to_bf16_array(_ptr(a), a.size, _ptr(out))
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def f32_to_e4m3(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint8)
    _load().oracle_f32_to_e4m3_array(_ptr(a), a.size, _ptr(out))
    return out


def e4m3_to_f32(codes: np.ndarray) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(codes.shape, dtype=np.float32)
    _load().oracle_e4m3_to_f32_array(_ptr(codes), codes.size, _ptr(out))
    return out


# --------------------------------------------------------------------------
# Layout / dispatch / combine
# --------------------------------------------------------------------------

def layout(expert_ids: np.ndarray, num_experts: int, align: int = 128):
    """Returns ``(expert_counts[E], ep_send_counts[E+1], expand_idx[BS*K], flags)``."""
    ids = _i32(expert_ids)
    assert ids.ndim == 2
    bs, k = ids.shape
    counts = np.zeros(num_experts, dtype=np.int32)
    send = np.zeros(num_experts + 1, dtype=np.int32)
    idx = np.zeros(bs * k, dtype=np.int32)
    flags = np.zeros(1, dtype=np.int32)
    rc = _load().oracle_layout(_ptr(ids), bs, k, num_experts, align, _ptr(counts), _ptr(send),
                               _ptr(idx), _ptr(flags))
    if rc != OK:
        raise OracleArgError(rc)
    return counts, send, idx, int(flags[0])


def dispatch_bf16(x_bits: np.ndarray, expert_ids: np.ndarray, expand_idx: np.ndarray,
                  ep_send_counts: np.ndarray, num_experts: int, capacity_rows: int,
                  out: np.ndarray | None = None):
    """``x_bits``: uint16 [BS, H] bf16 bit patterns.  Returns ``(expand_x, flags)``
    where ``expand_x`` is uint16 [capacity_rows, H], unwritten rows = sentinel."""
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    ids = _i32(expert_ids)
    bs, k = ids.shape
    hidden = x_bits.shape[1]
    if out is None:
        out = np.full((capacity_rows, hidden), SENTINEL_BF16, dtype=np.uint16)
    flags = np.zeros(1, dtype=np.int32)
    rc = _load().oracle_dispatch_bf16(_ptr(x_bits), hidden, bs, hidden, _ptr(ids),
                                      _ptr(_i32(expand_idx)), _ptr(_i32(ep_send_counts)), k,
                                      num_experts, _ptr(out), hidden, capacity_rows, _ptr(flags))
    if rc != OK:
        raise OracleArgError(rc)
    return out, int(flags[0])


def quantize_row_e4m3(x_row_bits: np.ndarray):
    """One token row (uint16 bf16 bits, length H) -> (codes uint8[H], scales f32[H/128])."""
    x_row_bits = np.ascontiguousarray(x_row_bits, dtype=np.uint16)
    hidden = x_row_bits.shape[0]
    q = np.empty(hidden, dtype=np.uint8)
    s = np.empty(hidden // 128, dtype=np.float32)
    _load().oracle_quantize_row_e4m3(_ptr(x_row_bits), hidden, _ptr(q), _ptr(s))
    return q, s


def dispatch_fp8(x_bits: np.ndarray, expert_ids: np.ndarray, expand_idx: np.ndarray,
                 ep_send_counts: np.ndarray, num_experts: int, capacity_rows: int):
    """Returns ``(codes uint8 [cap, H], scales f32 [cap, H/128], flags)``; unwritten
    rows hold the sentinels."""
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    ids = _i32(expert_ids)
    bs, k = ids.shape
    hidden = x_bits.shape[1]
    codes = np.full((capacity_rows, hidden), SENTINEL_FP8, dtype=np.uint8)
    scales = np.full((capacity_rows, max(hidden // 128, 1)), SENTINEL_SCALE, dtype=np.float32)
    q_tmp = np.empty(hidden, dtype=np.uint8)
    s_tmp = np.empty(max(hidden // 128, 1), dtype=np.float32)
    flags = np.zeros(1, dtype=np.int32)
    rc = _load().oracle_dispatch_fp8(_ptr(x_bits), hidden, bs, hidden, _ptr(ids),
                                     _ptr(_i32(expand_idx)), _ptr(_i32(ep_send_counts)), k,
                                     num_experts, _ptr(codes), hidden, capacity_rows,
                                     _ptr(scales), _ptr(flags), _ptr(q_tmp), _ptr(s_tmp))
    if rc != OK:
        raise OracleArgError(rc)
    return codes, scales, int(flags[0])


def combine(y_bits: np.ndarray, expert_ids: np.ndarray, expand_idx: np.ndarray,
            ep_send_counts: np.ndarray, expert_scales: np.ndarray,
            shared_bits: np.ndarray | None, num_experts: int):
    """``y_bits``: uint16 [capacity_rows, H]; ``shared_bits``: uint16 [BS, H] or None.
    Returns ``(x_out uint16 [BS, H], flags)``."""
    y_bits = np.ascontiguousarray(y_bits, dtype=np.uint16)
    ids = _i32(expert_ids)
    bs, k = ids.shape
    cap, hidden = y_bits.shape
    scales = np.ascontiguousarray(expert_scales, dtype=np.float32)
    if shared_bits is not None:
        shared_bits = np.ascontiguousarray(shared_bits, dtype=np.uint16)
    out = np.empty((bs, hidden), dtype=np.uint16)
    flags = np.zeros(1, dtype=np.int32)
    rc = _load().oracle_combine(_ptr(y_bits), hidden, cap, _ptr(ids), _ptr(_i32(expand_idx)),
                                _ptr(_i32(ep_send_counts)), _ptr(scales), _ptr(shared_bits),
                                hidden, bs, hidden, k, num_experts, _ptr(out), _ptr(flags))
    if rc != OK:
        raise OracleArgError(rc)
    return out, int(flags[0])


def combine_fp8(y_codes: np.ndarray, y_scales: np.ndarray, expert_ids: np.ndarray,
                expand_idx: np.ndarray, ep_send_counts: np.ndarray, expert_scales: np.ndarray,
                shared_bits: np.ndarray | None, num_experts: int):
    """``y_codes``: uint8 [capacity_rows, H] e4m3 codes; ``y_scales``: f32
    [capacity_rows, H/128].  Returns ``(x_out uint16 [BS, H], flags)``."""
    y_codes = np.ascontiguousarray(y_codes, dtype=np.uint8)
    y_scales = np.ascontiguousarray(y_scales, dtype=np.float32)
    ids = _i32(expert_ids)
    bs, k = ids.shape
    cap, hidden = y_codes.shape
    scales = np.ascontiguousarray(expert_scales, dtype=np.float32)
    if shared_bits is not None:
        shared_bits = np.ascontiguousarray(shared_bits, dtype=np.uint16)
    out = np.empty((bs, hidden), dtype=np.uint16)
    flags = np.zeros(1, dtype=np.int32)
    rc = _load().oracle_combine_fp8(_ptr(y_codes), hidden, cap, _ptr(y_scales), _ptr(ids),
                                    _ptr(_i32(expand_idx)), _ptr(_i32(ep_send_counts)),
                                    _ptr(scales), _ptr(shared_bits), hidden, bs, hidden, k,
                                    num_experts, _ptr(out), _ptr(flags))
    if rc != OK:
        raise OracleArgError(rc)
    return out, int(flags[0])


def splitmix64(seed: int, i: int) -> int:
    """Draw ``i`` of the SplitMix64 stream seeded with ``seed``."""
    return int(_load().oracle_splitmix64(seed & 0xFFFFFFFFFFFFFFFF, i))


def layout_replicated(expert_ids: np.ndarray, num_experts: int, replica_offsets: np.ndarray,
                      replica_thresholds: np.ndarray, seed: int, align: int = 128):
    """Returns ``(replica_ids[BS,K], replica_counts[P], ep_send_counts[P+1],
    expand_idx[BS*K], flags)``."""
    ids = _i32(expert_ids)
    bs, k = ids.shape
    off = _i32(replica_offsets)
    thr = np.ascontiguousarray(replica_thresholds, dtype=np.uint32)
    p = thr.size
    rep = np.zeros((bs, k), np.int32)
    counts = np.zeros(p, np.int32)
    send = np.zeros(p + 1, np.int32)
    idx = np.zeros(bs * k, np.int32)
    flags = np.zeros(1, np.int32)
    rc = _load().oracle_layout_replicated(_ptr(ids), bs, k, num_experts, _ptr(off), _ptr(thr), p,
                                          seed & 0xFFFFFFFFFFFFFFFF, align, _ptr(rep),
                                          _ptr(counts), _ptr(send), _ptr(idx), _ptr(flags))
    if rc != OK:
        raise OracleArgError(rc)
    return rep, counts, send, idx, int(flags[0])


def layout_ep(expert_ids: np.ndarray, num_experts: int, ep_world_size: int, align: int = 128):
    """Returns ``(expert_counts, ep_send_counts, rank_offsets[ws+1], expand_idx, flags)``."""
    ids = _i32(expert_ids)
    bs, k = ids.shape
    counts = np.zeros(num_experts, np.int32)
    send = np.zeros(num_experts + 1, np.int32)
    ranks = np.zeros(max(ep_world_size, 0) + 1, np.int32)
    idx = np.zeros(bs * k, np.int32)
    flags = np.zeros(1, np.int32)
    rc = _load().oracle_layout_ep(_ptr(ids), bs, k, num_experts, ep_world_size, align,
                                  _ptr(counts), _ptr(send), _ptr(ranks), _ptr(idx), _ptr(flags))
    if rc != OK:
        raise OracleArgError(rc)
    return counts, send, ranks, idx, int(flags[0])
