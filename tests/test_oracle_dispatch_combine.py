"""Pins for the oracle's dispatch (bf16, e4m3) and combine.

Dispatch: bijection + row equality against the definition (every real row is
the token row that maps to it, bit for bit; padding untouched).  FP8: the
closed-form e4m3 error bound, the "every non-zero block holds a +-448 code"
invariant, zero blocks, and the tolerance reading (relative error with a
subnormal floor, cosine in float64).  Combine: the identity-expert
round trip, one-hot gathers, an exactly representable worked example, the
unweighted shared row, and an float64 definition rounded once to bf16.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads


def small_case(bs=40, hidden=256, e=16, k=4, seed=5, align=8):
    rng = np.random.default_rng(seed)
    ids = np.argsort(rng.random((bs, e)), axis=1)[:, :k].astype(np.int32)
    x = workloads.bits(torch.randn(bs, hidden, generator=torch.Generator().manual_seed(seed)).to(
        torch.bfloat16))
    counts, send, idx, _ = oracle.layout(ids, e, align)
    cap = oracle.capacity(bs, k, e, align)
    return ids, x, counts, send, idx, cap


def slots_of(ids, send, idx):
    return send[ids.ravel()].astype(np.int64) + idx


# ---------------------------------------------------------------- dispatch bf16

def test_dispatch_bf16_bijection_and_rows():
    ids, x, counts, send, idx, cap = small_case()
    out, flags = oracle.dispatch_bf16(x, ids, idx, send, 16, cap)
    assert flags == 0
    bs, k = ids.shape
    slot = slots_of(ids, send, idx)
    tok = np.repeat(np.arange(bs), k)
    np.testing.assert_array_equal(out[slot], x[tok])
    written = np.zeros(cap, bool)
    written[slot] = True
    assert written.sum() == bs * k
    assert np.all(out[~written] == oracle.SENTINEL_BF16)
    # P2's checklist: expert ids recoverable from the slot ranges
    seg = np.searchsorted(send, slot, side="right") - 1
    np.testing.assert_array_equal(seg, ids.ravel())


def test_dispatch_guard_and_invalid_pairs():
    ids = np.array([[0, 1], [1, 9]], dtype=np.int32)
    x = np.arange(2 * 32, dtype=np.uint16).reshape(2, 32)
    send = np.array([0, 4, 8] + [8] * 8, dtype=np.int32)
    idx = np.array([0, 0, 1, -1], dtype=np.int32)
    # pairs: (0,0) -> row 0, (0,1) -> row 4, (1,0) -> row 5 = capacity (guard
    # hit, skipped), (1,1) has a negative index (skipped, no flag)
    out, flags = oracle.dispatch_bf16(x, ids, idx, send, 10, 5)
    assert flags == oracle.FLAG_GUARD
    np.testing.assert_array_equal(out[0], x[0])
    np.testing.assert_array_equal(out[4], x[0])
    assert np.all(out[1:4] == oracle.SENTINEL_BF16)


def test_dispatch_guard_flag():
    ids = np.array([[0, 1]], dtype=np.int32)
    x = np.ones((1, 32), dtype=np.uint16)
    send = np.array([0, 4, 8], dtype=np.int32)
    idx = np.array([0, 0], dtype=np.int32)
    out, flags = oracle.dispatch_bf16(x, ids, idx, send, 2, 4)  # slot 4 is out of range
    assert flags == oracle.FLAG_GUARD
    assert np.all(out[0] == 1)


# ---------------------------------------------------------------- fp8

def test_quantize_error_bound_and_448_invariant():
    rng = np.random.default_rng(2)
    hidden = 1024
    xf = np.concatenate([rng.standard_normal(hidden * 50) * 10.0 ** rng.integers(-4, 3),
                         rng.standard_normal(hidden * 50)])
    xb = oracle.f32_to_bf16_bits(xf.astype(np.float32)).reshape(-1, hidden)
    for row in xb:
        q, s = oracle.quantize_row_e4m3(row)
        xv = oracle.bf16_bits_to_f32(row).astype(np.float64)
        deq = oracle.e4m3_to_f32(q).astype(np.float64) * np.repeat(s.astype(np.float64), 128)
        sc = np.repeat(s.astype(np.float64), 128)
        err = np.abs(deq - xv)
        normal = np.abs(xv) >= 2.0 ** -6 * sc * (1 + 2 ** -20)
        # closed forms: 3 mantissa bits -> half-ulp relative 2^-4 for normals,
        # half the subnormal spacing 2^-9 for subnormals (plus the rounding of
        # x/s in binary32, far below these bounds)
        assert np.all(err[normal] <= 2.0 ** -4 * np.abs(xv[normal]) * (1 + 2 ** -20))
        assert np.all(err[~normal] <= 2.0 ** -10 * sc[~normal] * (1 + 2 ** -20))
        blocks = q.reshape(-1, 128)
        for b in range(blocks.shape[0]):
            if s[b] > 0:
                assert np.any((blocks[b] == 0x7E) | (blocks[b] == 0xFE))


def test_quantize_zero_block_and_scale_value():
    row = np.zeros(256, dtype=np.uint16)
    row[128 + 5] = oracle.f32_to_bf16_bits(np.array([-3.5], np.float32))[0]
    q, s = oracle.quantize_row_e4m3(row)
    assert s[0] == 0.0 and np.all(q[:128] == 0)
    assert s[1] == np.float32(3.5) / np.float32(448.0)
    assert q[128 + 5] == 0xFE  # -448
    assert np.all(np.delete(q[128:], 5) == 0x00)


def test_quantize_exact_power_of_two_block():
    # amax = 448 gives s = 1, so every code is e4m3(x) directly
    vals = np.concatenate([[448.0], np.linspace(-400, 400, 127)]).astype(np.float32)
    row = oracle.f32_to_bf16_bits(vals)
    q, s = oracle.quantize_row_e4m3(row)
    assert s[0] == 1.0
    np.testing.assert_array_equal(q, oracle.f32_to_e4m3(oracle.bf16_bits_to_f32(row)))


def fp8_tolerance_metrics(x_bits, q, s):
    """Relative error with a floor at the smallest normal (2^-6 * s), and
    per-row / global cosine, all in float64."""
    xv = oracle.bf16_bits_to_f32(x_bits).astype(np.float64)
    sc = np.repeat(s.astype(np.float64), 128, axis=-1)
    deq = oracle.e4m3_to_f32(q).astype(np.float64) * sc
    denom = np.maximum(np.abs(xv), 2.0 ** -6 * sc)
    with np.errstate(invalid="ignore", divide="ignore"):
        rel = np.where(denom > 0, np.abs(deq - xv) / np.where(denom > 0, denom, 1), 0.0)
    num = (deq * xv).sum(-1)
    den = np.sqrt((deq * deq).sum(-1) * (xv * xv).sum(-1))
    cos_rows = np.where(den > 0, num / np.where(den > 0, den, 1), 1.0)
    cos_all = (deq * xv).sum() / np.sqrt((deq * deq).sum() * (xv * xv).sum())
    return rel.max(), cos_rows.min(), cos_all


def test_fp8_tolerance_reading():
    x = workloads.bits(workloads.bf16_rows(64, 7168, seed=3))
    qs = [oracle.quantize_row_e4m3(r) for r in x]
    q = np.stack([a for a, _ in qs])
    s = np.stack([b for _, b in qs])
    rel, cmin, call = fp8_tolerance_metrics(x, q, s)
    assert rel <= 0.0625 * (1 + 1e-6) < 0.07
    assert cmin >= 0.999 and call >= 0.999


def test_dispatch_fp8_copies_are_identical():
    ids, x, counts, send, idx, cap = small_case(hidden=384)
    codes, scales, flags = oracle.dispatch_fp8(x, ids, idx, send, 16, cap)
    assert flags == 0
    bs, k = ids.shape
    slot = slots_of(ids, send, idx).reshape(bs, k)
    for t in range(bs):
        q, s = oracle.quantize_row_e4m3(x[t])
        for j in range(k):
            np.testing.assert_array_equal(codes[slot[t, j]], q)
            np.testing.assert_array_equal(scales[slot[t, j]], s)
    written = np.zeros(cap, bool)
    written[slot.ravel()] = True
    assert np.all(codes[~written] == oracle.SENTINEL_FP8)
    assert np.all(scales[~written] == oracle.SENTINEL_SCALE)


# ---------------------------------------------------------------- combine

def test_combine_identity_experts_round_trip():
    """Identity experts (y = dispatched rows), scales summing to 1, no shared
    row: the output is x bit for bit (the fp32 sum deviates from x by at most
    ~K*2^-23 relative, far inside half a bf16 ulp)."""
    for name in ("tiny",):
        w = workloads.WORKLOADS[name]
        inp = workloads.make(w)
        ids, sc = inp["expert_ids"], inp["expert_scales"]
        x = workloads.bits(inp["x"])
        counts, send, idx, _ = oracle.layout(ids, w.experts, w.align)
        cap = oracle.capacity(w.bs, w.topk, w.experts, w.align)
        y, _ = oracle.dispatch_bf16(x, ids, idx, send, w.experts, cap)
        out, flags = oracle.combine(y, ids, idx, send, sc, None, w.experts)
        assert flags == 0
        np.testing.assert_array_equal(out, x)
    ids, x, counts, send, idx, cap = small_case(bs=300, hidden=512, e=64, k=8)
    y, _ = oracle.dispatch_bf16(x, ids, idx, send, 64, cap)
    sc = workloads.scales(300, 8, seed=11)
    out, _ = oracle.combine(y, ids, idx, send, sc, None, 64)
    xf = oracle.bf16_bits_to_f32(x)
    of = oracle.bf16_bits_to_f32(out)
    np.testing.assert_array_equal(of, xf)


def test_combine_one_hot_is_a_gather():
    ids, x, counts, send, idx, cap = small_case()
    rng = np.random.default_rng(9)
    y = oracle.f32_to_bf16_bits(rng.standard_normal((cap, x.shape[1])).astype(np.float32))
    bs, k = ids.shape
    pick = rng.integers(0, k, bs)
    sc = np.zeros((bs, k), np.float32)
    sc[np.arange(bs), pick] = 1.0
    out, _ = oracle.combine(y, ids, idx, send, sc, None, 16)
    slot = slots_of(ids, send, idx).reshape(bs, k)
    expect = y[slot[np.arange(bs), pick]]
    # bit-exact except that -0 inputs come out +0 (the chain starts from +0)
    np.testing.assert_array_equal(oracle.bf16_bits_to_f32(out), oracle.bf16_bits_to_f32(expect))


def test_combine_shared_row_is_unweighted():
    ids, x, counts, send, idx, cap = small_case()
    bs, k = ids.shape
    y = np.zeros((cap, x.shape[1]), np.uint16)
    sc = np.full((bs, k), 7.0, np.float32)
    out, _ = oracle.combine(y, ids, idx, send, sc, x, 16)
    np.testing.assert_array_equal(oracle.bf16_bits_to_f32(out), oracle.bf16_bits_to_f32(x))


def test_combine_exact_worked_example():
    """Small-integer rows and dyadic scales: every partial sum is exact in
    fp32, so the result is the rational formula evaluated by hand."""
    hidden, e, k = 32, 4, 3
    ids = np.array([[2, 0, 3], [1, 2, 0]], dtype=np.int32)
    counts, send, idx, _ = oracle.layout(ids, e, 1)
    cap = int(send[-1])
    y = np.zeros((cap, hidden), np.float32)
    for r in range(cap):
        y[r] = (np.arange(hidden) % 7) - 3 + r  # small integers, row-dependent
    sc = np.array([[1.0, 0.5, 0.25], [0.125, 2.0, -1.0]], np.float32)
    shared = (np.arange(2 * hidden).reshape(2, hidden) % 5 - 2).astype(np.float32)
    out, _ = oracle.combine(oracle.f32_to_bf16_bits(y), ids, idx, send, sc,
                            oracle.f32_to_bf16_bits(shared), e)
    slot = slots_of(ids, send, idx).reshape(2, k)
    for t in range(2):
        for h in range(hidden):
            v = sum(Fraction(float(sc[t, j])) * Fraction(float(y[slot[t, j], h]))
                    for j in range(k)) + Fraction(float(shared[t, h]))
            assert oracle.bf16_bits_to_f32(out[t:t + 1, h:h + 1])[0, 0] == float(v)


def test_combine_against_float64_definition():
    """Float64 evaluation of the formula rounded once to bf16 differs from the
    fp32 chain by at most one bf16 ulp, except where the sum cancels."""
    ids, x, counts, send, idx, cap = small_case(bs=200, hidden=512, e=32, k=8, seed=4)
    rng = np.random.default_rng(4)
    y = oracle.f32_to_bf16_bits(rng.standard_normal((cap, 512)).astype(np.float32))
    shared = oracle.f32_to_bf16_bits(rng.standard_normal((200, 512)).astype(np.float32))
    sc = workloads.scales(200, 8, seed=4)
    out, _ = oracle.combine(y, ids, idx, send, sc, shared, 32)
    slot = slots_of(ids, send, idx).reshape(200, 8)
    yf = oracle.bf16_bits_to_f32(y).astype(np.float64)
    ref = (sc.astype(np.float64)[:, :, None] * yf[slot]).sum(1) + oracle.bf16_bits_to_f32(
        shared).astype(np.float64)
    ref_b = oracle.f32_to_bf16_bits(ref.astype(np.float32))
    ob = out.astype(np.int32)
    rb = ref_b.astype(np.int32)
    same_sign = (ob >> 15) == (rb >> 15)
    ulp = np.abs((ob & 0x7FFF) - (rb & 0x7FFF))
    mag = np.abs(ref)
    terms = (np.abs(sc.astype(np.float64)[:, :, None] * yf[slot]).sum(1)
             + np.abs(oracle.bf16_bits_to_f32(shared)))
    well_conditioned = mag > 2.0 ** -6 * terms
    assert np.all(ulp[well_conditioned & same_sign] <= 1)
    assert well_conditioned.mean() > 0.95


def test_combine_skips_invalid_pairs():
    ids = np.array([[0, 1]], dtype=np.int32)
    y = oracle.f32_to_bf16_bits(np.array([[1.0] * 32, [2.0] * 32], np.float32))
    send = np.array([0, 1, 2], dtype=np.int32)
    sc = np.array([[1.0, 1.0]], np.float32)
    out, flags = oracle.combine(y, ids, np.array([0, -1], np.int32), send, sc, None, 2)
    assert np.all(oracle.bf16_bits_to_f32(out) == 1.0) and flags == 0
    out, flags = oracle.combine(y, ids, np.array([0, 5], np.int32), send, sc, None, 2)
    assert np.all(oracle.bf16_bits_to_f32(out) == 1.0) and flags == oracle.FLAG_GUARD


@pytest.mark.parametrize("hidden,dtype,code", [(0, 0, 1), (48, 0, 1), (96, 1, 1), (128, 1, 0),
                                               (32, 0, 0), (7168, 0, 0), (7168, 1, 0), (64, 2, 3)])
def test_row_rules(hidden, dtype, code):
    assert oracle.check_row_args(hidden, dtype) == code
