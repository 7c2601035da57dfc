"""Pins for the oracle's quantised-transfer combine (e4m3 expert rows with one
fp32 scale per 128 channels, dequantised term by term).

Checked against: torch's float8_e4m3fn decode and bfloat16 cast (library
routines) for one-hot weights over every code; an exactly representable
worked example; a float64 evaluation of the formula; and the round trip
through the oracle's own e4m3 dispatch.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads


def torch_decode(codes: np.ndarray) -> np.ndarray:
    return torch.from_numpy(codes.astype(np.uint8)).view(torch.float8_e4m3fn).float().numpy()


def torch_bf16_bits(a: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)


def identity_layout(bs, k, e):
    ids = np.array([[(t * k + j) % e for j in range(k)] for t in range(bs)], np.int32)
    counts, send, idx, _ = oracle.layout(ids, e, 1)
    return ids, send, idx


def test_one_hot_every_code():
    """Row r holds code r % 256 everywhere; one-hot weights pick one row per
    token, so each output is bf16(decode(code) * s)."""
    hidden = 128
    cap = 256
    codes = np.repeat(np.arange(256, dtype=np.uint8)[:, None], hidden, 1)
    scales = np.full((cap, 1), 0.37, np.float32)
    bs, k, e = 256, 1, 256
    ids = np.arange(256, dtype=np.int32).reshape(bs, 1)
    counts, send, idx, _ = oracle.layout(ids, e, 1)
    out, flags = oracle.combine_fp8(codes, scales, ids, idx, send, np.ones((bs, k), np.float32),
                                    None, e)
    ref_f32 = (torch_decode(np.arange(256)) * np.float32(0.37)).astype(np.float32)
    ref = torch_bf16_bits(ref_f32)
    finite = np.isfinite(ref_f32)
    # compared as values: the chain starts from +0, so code 0x80 (-0) gives +0
    np.testing.assert_array_equal(oracle.bf16_bits_to_f32(out[finite, 0]),
                                  oracle.bf16_bits_to_f32(ref[finite]))
    assert np.all(np.isnan(oracle.bf16_bits_to_f32(out[~finite, 0])))
    assert flags == 0


def test_exact_worked_example():
    # integer codes (e4m3 holds 0..16 exactly), power-of-two scales and dyadic
    # weights keep every partial sum exact in fp32; only the final bf16
    # rounding applies
    hidden, k, e = 256, 3, 5
    ids = np.array([[4, 0, 2], [1, 3, 4]], np.int32)
    counts, send, idx, _ = oracle.layout(ids, e, 1)
    cap = int(send[-1])
    ints = (np.arange(cap * hidden).reshape(cap, hidden) % 17 - 8).astype(np.float32)
    codes = torch.from_numpy(ints).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    scales = np.array([[0.5, 2.0]] * cap, np.float32)
    scales[1] = [0.25, 4.0]
    w = np.array([[1.0, 0.5, -0.25], [0.125, 2.0, 1.0]], np.float32)
    shared = (np.arange(2 * hidden).reshape(2, hidden) % 5 - 2).astype(np.float32)
    out, _ = oracle.combine_fp8(codes, scales, ids, idx, send, w,
                                oracle.f32_to_bf16_bits(shared), e)
    slot = send[ids.ravel()].astype(np.int64).reshape(2, k) + idx.reshape(2, k)
    for t in range(2):
        for h in range(0, hidden, 7):
            v = sum(Fraction(float(w[t, j])) * Fraction(float(ints[slot[t, j], h]))
                    * Fraction(float(scales[slot[t, j], h // 128])) for j in range(k))
            v += Fraction(float(shared[t, h]))
            # the fp32 sum is exact (checked), the output is its bf16 rounding
            assert float(np.float32(float(v))) == float(v)
            expect = torch_bf16_bits(np.array([float(v)], np.float32))[0]
            assert out[t, h] == expect


def test_against_float64_definition():
    rng = np.random.default_rng(12)
    bs, hidden, e, k = 150, 512, 32, 8
    ids = np.argsort(rng.random((bs, e)), axis=1)[:, :k].astype(np.int32)
    counts, send, idx, _ = oracle.layout(ids, e, 128)
    cap = oracle.capacity(bs, k, e, 128)
    codes = rng.integers(0, 256, (cap, hidden), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x38          # no NaN codes
    scales = rng.uniform(1e-3, 1e-2, (cap, hidden // 128)).astype(np.float32)
    w = workloads.scales(bs, k, seed=5)
    shared = oracle.f32_to_bf16_bits(rng.standard_normal((bs, hidden)).astype(np.float32))
    out, _ = oracle.combine_fp8(codes, scales, ids, idx, send, w, shared, e)
    slot = send[ids.ravel()].astype(np.int64).reshape(bs, k) + idx.reshape(bs, k)
    deq = torch_decode(codes).astype(np.float64) * np.repeat(scales.astype(np.float64), 128, 1)
    terms = w.astype(np.float64)[:, :, None] * deq[slot]
    ref = terms.sum(1) + oracle.bf16_bits_to_f32(shared).astype(np.float64)
    ref_b = torch_bf16_bits(ref.astype(np.float32)).astype(np.int32)
    ob = out.astype(np.int32)
    well = np.abs(ref) > 2.0 ** -6 * (np.abs(terms).sum(1) + np.abs(
        oracle.bf16_bits_to_f32(shared)))
    same_sign = (ob >> 15) == (ref_b >> 15)
    assert np.all(np.abs((ob & 0x7FFF) - (ref_b & 0x7FFF))[well & same_sign] <= 1)
    assert well.mean() > 0.95


def test_round_trip_through_fp8_dispatch():
    """Identity experts on the e4m3 path: y is the oracle's own dispatched
    codes / scales, weights sum to 1, no shared row.  Every output is within
    one bf16 ulp of the dequantised token (float64 reference)."""
    w = workloads.WORKLOADS["tiny"]
    inp = workloads.make(w)
    ids, sc = inp["expert_ids"], inp["expert_scales"]
    x = workloads.bits(inp["x"])
    counts, send, idx, _ = oracle.layout(ids, w.experts, w.align)
    cap = oracle.capacity(w.bs, w.topk, w.experts, w.align)
    codes, scales, _ = oracle.dispatch_fp8(x, ids, idx, send, w.experts, cap)
    out, flags = oracle.combine_fp8(codes, scales, ids, idx, send, sc, None, w.experts)
    assert flags == 0
    qs = [oracle.quantize_row_e4m3(r) for r in x]
    deq = np.stack([torch_decode(q).astype(np.float64) * np.repeat(s.astype(np.float64), 128)
                    for q, s in qs])
    ref_b = torch_bf16_bits(deq.astype(np.float32)).astype(np.int32)
    assert np.abs(out.astype(np.int32) - ref_b).max() <= 1


def test_skipped_pairs_and_guard():
    ids = np.array([[0, 1]], np.int32)
    codes = np.full((2, 128), 0x38, np.uint8)   # 1.0
    scales = np.ones((2, 1), np.float32)
    send = np.array([0, 1, 2], np.int32)
    w = np.ones((1, 2), np.float32)
    out, f = oracle.combine_fp8(codes, scales, ids, np.array([0, -1], np.int32), send, w, None, 2)
    assert np.all(oracle.bf16_bits_to_f32(out) == 1.0) and f == 0
    out, f = oracle.combine_fp8(codes, scales, ids, np.array([0, 3], np.int32), send, w, None, 2)
    assert np.all(oracle.bf16_bits_to_f32(out) == 1.0) and f == oracle.FLAG_GUARD


@pytest.mark.parametrize("hidden", [0, 32, 96])
def test_rejects_hidden_not_multiple_of_128(hidden):
    ids = np.zeros((1, 1), np.int32)
    with pytest.raises(oracle.OracleArgError):
        oracle.combine_fp8(np.zeros((1, max(hidden, 1)), np.uint8)[:, :hidden],
                           np.zeros((1, 1), np.float32), ids, np.zeros(1, np.int32),
                           np.zeros(2, np.int32), np.ones((1, 1), np.float32), None, 1)
