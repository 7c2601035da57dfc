"""Pins for the oracle's number formats against library conversions.

bf16 narrowing is checked against torch's float32 -> bfloat16 cast and e4m3fn
against torch's float8_e4m3fn cast (both round to nearest even); the whole
e4m3 code space is decoded and re-encoded.  torch maps magnitudes above the
midpoint 464 to NaN while the oracle saturates to 448, so the saturation
rule is pinned by closed form instead.
"""

import numpy as np
import torch

import oracle


def torch_bf16_bits(a: np.ndarray) -> np.ndarray:
    return torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(
        np.uint16)


def torch_e4m3(a: np.ndarray) -> np.ndarray:
    return torch.from_numpy(a.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_bf16_widening_is_exact():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    f = oracle.bf16_bits_to_f32(bits)
    t = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    finite = np.isfinite(t)
    np.testing.assert_array_equal(f[finite], t[finite])
    assert np.all(np.isnan(f[~np.isfinite(t) & np.isnan(t)]))


def test_bf16_rne_all_midpoints_and_neighbours():
    # every finite bf16 value b; probe b + d*ulp/2^16 for d in a set that hits
    # the exact midpoint, just below, just above and the extremes
    hi = np.arange(1 << 16, dtype=np.uint32)
    hi = hi[((hi >> 7) & 0xFF) != 0xFF]  # finite only
    lows = np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF], dtype=np.uint32)
    u = (hi[:, None] << 16 | lows[None, :]).ravel()
    f = u.view(np.float32)
    ours = oracle.f32_to_bf16_bits(f)
    ref = torch_bf16_bits(f)
    np.testing.assert_array_equal(ours, ref)


def test_bf16_rne_random_and_special():
    rng = np.random.default_rng(0)
    u = rng.integers(0, 1 << 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    f = u.view(np.float32)
    f = f[np.isfinite(f)]
    np.testing.assert_array_equal(oracle.f32_to_bf16_bits(f), torch_bf16_bits(f))
    special = np.array([0.0, -0.0, np.inf, -np.inf, 3.4028235e38, -3.4028235e38, 1e-45, -1e-45],
                       dtype=np.float32)
    np.testing.assert_array_equal(oracle.f32_to_bf16_bits(special), torch_bf16_bits(special))
    assert np.isnan(oracle.bf16_bits_to_f32(oracle.f32_to_bf16_bits(np.array([np.nan],
                                                                             np.float32))))[0]


def test_e4m3_decode_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_to_f32(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).float().numpy()
    nan = np.isnan(ref)
    assert set(np.nonzero(nan)[0].tolist()) == {0x7F, 0xFF}
    assert np.all(np.isnan(ours[nan]))
    np.testing.assert_array_equal(ours[~nan], ref[~nan])
    # named values of the format
    assert ours[0x7E] == 448.0 and ours[0xFE] == -448.0
    assert ours[0x08] == 2.0 ** -6 and ours[0x01] == 2.0 ** -9
    assert ours[0x38] == 1.0


def test_e4m3_encode_roundtrips_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = oracle.e4m3_to_f32(codes)
    np.testing.assert_array_equal(oracle.f32_to_e4m3(vals), codes)


def test_e4m3_encode_midpoints_ties_to_even():
    codes = np.array([c for c in range(0x7E)], dtype=np.uint8)  # non-negative finite, ascending
    vals = oracle.e4m3_to_f32(codes).astype(np.float64)
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)  # exact in float32
    assert np.all(mids.astype(np.float64) == (vals[:-1] + vals[1:]) / 2)
    for sgn in (1.0, -1.0):
        m = (sgn * mids).astype(np.float32)
        ours = oracle.f32_to_e4m3(m)
        np.testing.assert_array_equal(ours, torch_e4m3(m))
        # ties go to the even code
        assert np.all((ours & 1) == 0)
        # one float32 ulp either side of the midpoint goes to the neighbours
        lo = np.nextafter(m, np.float32(0)).astype(np.float32)
        hi = np.nextafter(m, np.float32(sgn * np.inf)).astype(np.float32)
        np.testing.assert_array_equal(oracle.f32_to_e4m3(lo), torch_e4m3(lo))
        np.testing.assert_array_equal(oracle.f32_to_e4m3(hi), torch_e4m3(hi))


def test_e4m3_encode_random_in_range():
    rng = np.random.default_rng(1)
    a = np.concatenate([
        rng.uniform(-464, 464, 500_000),
        rng.standard_normal(500_000) * 0.01,
        rng.standard_normal(200_000) * 2.0 ** -8,
    ]).astype(np.float32)
    np.testing.assert_array_equal(oracle.f32_to_e4m3(a), torch_e4m3(a))


def test_e4m3_every_bf16_value_in_range():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    f = oracle.bf16_bits_to_f32(bits)
    f = f[np.isfinite(f) & (np.abs(f) <= 464)]
    np.testing.assert_array_equal(oracle.f32_to_e4m3(f), torch_e4m3(f))


def test_e4m3_saturation_closed_form():
    big = np.array([464.0001, 480.0, 1e6, 3.4e38, np.inf], dtype=np.float32)
    assert np.all(oracle.f32_to_e4m3(big) == 0x7E)
    assert np.all(oracle.f32_to_e4m3(-big) == 0xFE)
    assert oracle.f32_to_e4m3(np.array([np.nan], np.float32))[0] == 0x7F
    # signed zero and values that round to zero keep their sign
    assert oracle.f32_to_e4m3(np.array([-0.0, -2.0 ** -11], np.float32)).tolist() == [0x80, 0x80]
    assert oracle.f32_to_e4m3(np.array([0.0, 2.0 ** -11], np.float32)).tolist() == [0x00, 0x00]
