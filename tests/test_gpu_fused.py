"""GPU parity of moe_dispatch_fused (layout + dispatch in one call) against
the oracle's layout and bf16 dispatch.

Bars as for the separate calls: counts, offsets, ranks and status bit-exact;
the whole dispatched buffer bit-exact, including padding rows the call must
leave untouched (pre-filled with the oracle's sentinel) and canary rows past
capacity.  Batches of at most 2048 pairs take the one-launch kernels (bf16 and e4m3;
e4m3 codes and scales bit-exact against the oracle's quantiser); larger
batches take the layout + dispatch launches and, like the separate calls,
must give the oracle's whole buffer.
"""

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

DEV = "cuda"


def random_ids(rng, bs, e, k):
    return np.argsort(rng.random((bs, e)), axis=1)[:, :k].astype(np.int32)


def random_bf16(rng, shape):
    return oracle.f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32))


def to_dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def bits_of(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def run_fused(ids, x_bits, e, align, cap, canary_rows=0):
    import combine_moe_dispatch_layout_amd as moe
    bs, h = x_bits.shape
    buf = torch.full((cap + canary_rows, h), oracle.SENTINEL_BF16, dtype=torch.int16,
                     device=DEV).view(torch.bfloat16)
    ex = buf[:cap] if cap > 0 else buf[:0]
    lay, _ = moe.moe_dispatch_fused(to_dev_bf16(x_bits), torch.from_numpy(ids).to(DEV), e, align,
                                    expand_x=ex, capacity_rows=cap)
    torch.cuda.synchronize()
    return (lay.expert_counts.cpu().numpy(), lay.ep_send_counts.cpu().numpy(),
            lay.expand_idx.cpu().numpy(), int(lay.status.cpu()[0]), bits_of(buf))


def check_against_oracle(ids, x_bits, e, align, cap=None, canary_rows=0):
    bs, k = ids.shape
    if cap is None:
        cap = oracle.capacity(bs, k, e, align)
    c, s, r, f = oracle.layout(ids, e, align)
    ref_x, f2 = oracle.dispatch_bf16(x_bits, ids, r, s, e, cap)
    gc, gs, gr, gf, buf = run_fused(ids, x_bits, e, align, cap, canary_rows)
    np.testing.assert_array_equal(gc, c)
    np.testing.assert_array_equal(gs, s)
    np.testing.assert_array_equal(gr, r)
    assert gf == (f | f2), (gf, f, f2)
    np.testing.assert_array_equal(buf[:cap], ref_x)
    assert np.all(buf[cap:] == oracle.SENTINEL_BF16)  # nothing past capacity
    return f | f2


@pytest.mark.parametrize("bs,h,e,k,align", [
    (1, 32, 1, 1, 128), (7, 64, 3, 2, 1), (16, 128, 8, 2, 128), (128, 7168, 256, 8, 128),
    (100, 256, 512, 16, 128), (2048, 32, 64, 1, 128), (128, 4096, 64, 16, 128),
    (255, 1056, 40, 8, 64), (33, 256, 512, 3, 1024),
])
def test_one_launch_matches_the_oracle(bs, h, e, k, align):
    rng = np.random.default_rng(bs * 31 + k)
    ids = random_ids(rng, bs, e, k)
    assert check_against_oracle(ids, random_bf16(rng, (bs, h)), e, align) == 0


def test_one_launch_hot_expert_and_repeated_and_bad_ids():
    rng = np.random.default_rng(5)
    bs, h, e, k = 200, 512, 32, 8
    ids = np.tile(np.array([3, 9, 0, 31, 7, 12, 20, 5], np.int32), (bs, 1))   # one hot set
    assert check_against_oracle(ids, random_bf16(rng, (bs, h)), e, 128) == 0
    ids = random_ids(rng, bs, e, k)
    ids[::5, -1] = ids[::5, 0]                                                # repeats
    assert check_against_oracle(ids, random_bf16(rng, (bs, h)), e, 128) == oracle.FLAG_DUP_ID
    ids = random_ids(rng, bs, e, k)
    bad = rng.random(ids.shape) < 0.05
    ids[bad] = rng.choice([-1, e, e + 5, -700], size=int(bad.sum()))
    f = check_against_oracle(ids, random_bf16(rng, (bs, h)), e, 128)
    assert f & oracle.FLAG_ID_RANGE


def test_one_launch_guard_skips_rows_beyond_capacity():
    rng = np.random.default_rng(6)
    bs, h, e, k = 300, 256, 16, 4
    ids = random_ids(rng, bs, e, k)
    full = int(oracle.layout(ids, e, 128)[1][-1])
    f = check_against_oracle(ids, random_bf16(rng, (bs, h)), e, 128, cap=full - 200,
                             canary_rows=64)
    assert f & oracle.FLAG_GUARD
    check_against_oracle(ids, random_bf16(rng, (bs, h)), e, 128, cap=0, canary_rows=8)


def test_two_launch_paths_equal_the_separate_calls():
    """The separate layout + dispatch calls and moe_dispatch_fused, bf16 and
    e4m3, into sentinel-filled buffers: both give the oracle's layout and
    the oracle's whole dispatched buffer (e4m3 codes and scales of every
    row, padding rows untouched)."""
    import combine_moe_dispatch_layout_amd as moe
    rng = np.random.default_rng(7)
    for bs, h, e, k, dtype in [(4097, 256, 64, 1, "bf16"), (700, 512, 64, 8, "bf16"),
                               (100, 1024, 32, 4, "fp8"), (600, 256, 16, 8, "fp8"),
                               (128, 7168, 256, 8, "fp8"), (1500, 7168, 256, 8, "fp8")]:
        ids_h = random_ids(rng, bs, e, k)
        x_bits = random_bf16(rng, (bs, h))
        ids = torch.from_numpy(ids_h).to(DEV)
        x = to_dev_bf16(x_bits)
        cap = moe.moe_dispatch_capacity(bs, k, e, 128)
        c, s, r, f = oracle.layout(ids_h, e, 128)
        assert f == 0

        def buffers():
            if dtype == "bf16":
                return (torch.full((cap, h), oracle.SENTINEL_BF16, dtype=torch.int16,
                                   device=DEV).view(torch.bfloat16), None)
            return (torch.full((cap, h), oracle.SENTINEL_FP8, dtype=torch.uint8, device=DEV),
                    torch.full((cap, h // 128), oracle.SENTINEL_SCALE, dtype=torch.float32,
                               device=DEV))

        sep = moe.moe_dispatch_layout(ids, e, 128)
        sx, ss = buffers()
        moe.moe_dispatch(x, ids, sep.expand_idx, sep.ep_send_counts, e, capacity_rows=cap,
                         out_dtype=dtype, expand_x=sx, quant_scales=ss, status=sep.status)
        fx, fs = buffers()
        fused = moe.moe_dispatch_fused(x, ids, e, 128, capacity_rows=cap, out_dtype=dtype,
                                       expand_x=fx, quant_scales=fs)
        torch.cuda.synchronize()
        for lay in (sep, fused[0]):
            np.testing.assert_array_equal(lay.expert_counts.cpu().numpy(), c)
            np.testing.assert_array_equal(lay.ep_send_counts.cpu().numpy(), s)
            np.testing.assert_array_equal(lay.expand_idx.cpu().numpy(), r)
            assert int(lay.status.cpu()[0]) == 0
        if dtype == "bf16":
            ref, f2 = oracle.dispatch_bf16(x_bits, ids_h, r, s, e, cap)
            assert f2 == 0
            np.testing.assert_array_equal(bits_of(sx), ref)
            np.testing.assert_array_equal(bits_of(fx), ref)
        else:
            ref_q, ref_s, f2 = oracle.dispatch_fp8(x_bits, ids_h, r, s, e, cap)
            assert f2 == 0
            for q, sc in ((sx, ss), (fx, fs)):
                np.testing.assert_array_equal(q.cpu().numpy(), ref_q)
                np.testing.assert_array_equal(sc.cpu().numpy().view(np.uint32),
                                              ref_s.view(np.uint32))


@pytest.mark.parametrize("bs,h,e,k,align", [
    (300, 1056, 40, 8, 128),   # 2400 pairs; 132 vectors per row: ragged last 64-thread chunk
    (700, 512, 64, 8, 128),
    (1024, 7168, 256, 8, 128), # the prefill row width
    (5000, 32, 8, 1, 128),     # rows of 4 vectors: most threads of each workgroup idle
    (300, 256, 512, 16, 128),  # widest top-K, most experts
    (1001, 96, 40, 3, 64),     # odd K: tokens straddle the ranking workgroups' ranges
    (900, 128, 33, 5, 1),      # unpadded segments
])
def test_two_launch_path_matches_the_oracle(bs, h, e, k, align):
    """Batches above 2048 pairs with contiguous rows: the layout launches
    read every row ahead and the scatter runs in its cache-resident launch
    shape (64-thread workgroups, LDS-capped occupancy)."""
    rng = np.random.default_rng(bs + h)
    ids = random_ids(rng, bs, e, k)
    assert check_against_oracle(ids, random_bf16(rng, (bs, h)), e, align) == 0


@pytest.mark.parametrize("bs", [17554,    # 240 MiB of rows less 4 KB: every row read ahead
                                17555])   # just over: the first 128 MiB read ahead, the
                                          # scatter in its shape for rows from HBM
def test_two_launch_path_at_the_read_ahead_limit(bs):
    """The ranking launch reads all of x ahead up to 240 MiB and only the
    first 128 MiB of a larger x; on both sides of that limit the whole
    buffer equals the oracle's."""
    rng = np.random.default_rng(bs)
    h, e, k = 7168, 64, 2
    ids = random_ids(rng, bs, e, k)
    assert check_against_oracle(ids, random_bf16(rng, (bs, h)), e, 128) == 0


def test_two_launch_path_guard_and_hot_experts():
    rng = np.random.default_rng(9)
    bs, h, e, k = 700, 256, 16, 8
    ids = random_ids(rng, bs, e, k)
    m_pad = int(oracle.layout(ids, e, 128)[1][-1])   # padded rows the layout uses
    f = check_against_oracle(ids, random_bf16(rng, (bs, h)), e, 128, cap=m_pad - 200,
                             canary_rows=64)
    assert f & oracle.FLAG_GUARD
    hot = np.tile(np.arange(k, dtype=np.int32), (bs, 1))   # every token to experts 0..7
    assert check_against_oracle(hot, random_bf16(rng, (bs, h)), e, 128) == 0


def test_two_launch_path_strided_rows():
    """Rows with a stride beyond the row width are not read ahead, so the
    scatter keeps its full-occupancy shape; results as for contiguous rows."""
    import combine_moe_dispatch_layout_amd as moe
    rng = np.random.default_rng(10)
    bs, h, e, k = 600, 512, 64, 8
    ids = random_ids(rng, bs, e, k)
    wide = random_bf16(rng, (bs, h + 64))
    x = to_dev_bf16(wide)[:, :h]
    cap = oracle.capacity(bs, k, e, 128)
    c, s, r, f = oracle.layout(ids, e, 128)
    ref_x, _ = oracle.dispatch_bf16(np.ascontiguousarray(wide[:, :h]), ids, r, s, e, cap)
    buf = torch.full((cap, h), oracle.SENTINEL_BF16, dtype=torch.int16,
                     device=DEV).view(torch.bfloat16)
    lay, _ = moe.moe_dispatch_fused(x, torch.from_numpy(ids).to(DEV), e, 128, expand_x=buf,
                                    capacity_rows=cap)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(lay.expand_idx.cpu().numpy(), r)
    np.testing.assert_array_equal(bits_of(buf), ref_x)


def test_empty_batch_writes_zero_layout():
    import combine_moe_dispatch_layout_amd as moe
    x = torch.empty((0, 128), dtype=torch.bfloat16, device=DEV)
    ids = torch.empty((0, 4), dtype=torch.int32, device=DEV)
    lay, ex = moe.moe_dispatch_fused(x, ids, 16, 128, capacity_rows=0)
    torch.cuda.synchronize()
    assert int(lay.expert_counts.abs().sum()) == 0
    assert int(lay.ep_send_counts.abs().sum()) == 0
    assert int(lay.status.cpu()[0]) == 0


def test_zero_capacity_writes_nothing_and_flags_every_pair():
    import combine_moe_dispatch_layout_amd as moe
    rng = np.random.default_rng(8)
    ids = torch.from_numpy(random_ids(rng, 20, 8, 2)).to(DEV)
    x = to_dev_bf16(random_bf16(rng, (20, 256)))
    lay = moe.moe_dispatch_layout(ids, 8, 128)
    for dtype in ("bf16", "fp8"):
        st = torch.zeros(1, dtype=torch.int32, device=DEV)
        moe.moe_dispatch(x, ids, lay.expand_idx, lay.ep_send_counts, 8, capacity_rows=0,
                         out_dtype=dtype, status=st)
        torch.cuda.synchronize()
        assert int(st.cpu()[0]) == oracle.FLAG_GUARD


@pytest.mark.parametrize("bs,h,e,k,align", [
    (1, 128, 1, 1, 128), (16, 128, 8, 2, 128), (128, 7168, 256, 8, 128), (100, 512, 512, 16, 1),
    (2048, 128, 64, 1, 128), (37, 4224, 40, 8, 64),
])
def test_one_launch_e4m3_matches_the_oracle(bs, h, e, k, align):
    import combine_moe_dispatch_layout_amd as moe
    rng = np.random.default_rng(bs * 13 + k)
    ids = random_ids(rng, bs, e, k)
    x_bits = random_bf16(rng, (bs, h))
    x_bits[0, :128] = 0                                  # an all-zero block
    cap = oracle.capacity(bs, k, e, align)
    c, s, r, f = oracle.layout(ids, e, align)
    ref_codes, ref_scales, f2 = oracle.dispatch_fp8(x_bits, ids, r, s, e, cap)
    codes = torch.full((cap, h), oracle.SENTINEL_FP8, dtype=torch.uint8, device=DEV)
    scales = torch.full((cap, h // 128), oracle.SENTINEL_SCALE, dtype=torch.float32, device=DEV)
    lay, _, _ = moe.moe_dispatch_fused(to_dev_bf16(x_bits), torch.from_numpy(ids).to(DEV), e,
                                       align, capacity_rows=cap, out_dtype="fp8", expand_x=codes,
                                       quant_scales=scales)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(lay.expert_counts.cpu().numpy(), c)
    np.testing.assert_array_equal(lay.ep_send_counts.cpu().numpy(), s)
    np.testing.assert_array_equal(lay.expand_idx.cpu().numpy(), r)
    assert int(lay.status.cpu()[0]) == (f | f2) == 0
    np.testing.assert_array_equal(codes.cpu().numpy(), ref_codes)
    np.testing.assert_array_equal(scales.cpu().numpy().view(np.uint32),
                                  ref_scales.view(np.uint32))
