"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars: layout, ranks and dispatched bf16 rows bit-exact; e4m3 codes and scales
bit-exact (both sides decide each code in fp32 with a correctly rounded
division and round-to-nearest-even); combine within 1 bf16 ulp of the oracle
(identical fp32 FMA order, so 0 is expected and asserted as well).  Small
cases compare every element, including the untouched padding rows; the
full-size workloads compare the whole layout, every dispatched row of the
separate and the fused call (e4m3: the whole buffer against the oracle's;
bf16: each row against its token's and every padding row against the
sentinel) and every combined token against the oracle.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def lib():
    import combine_moe_dispatch_layout_amd as moe
    moe.load_library()
    assert torch.cuda.is_available()
    return moe


def moe_mod():
    import combine_moe_dispatch_layout_amd as moe
    return moe


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def random_ids(rng, bs, e, k):
    return np.argsort(rng.random((bs, e)), axis=1)[:, :k].astype(np.int32)


def random_bf16(rng, shape):
    return oracle.f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32))


def gpu_layout(ids, e, align):
    moe = moe_mod()
    lay = moe.moe_dispatch_layout(dev(ids), e, align)
    torch.cuda.synchronize()
    return (lay.expert_counts.cpu().numpy(), lay.ep_send_counts.cpu().numpy(),
            lay.expand_idx.cpu().numpy(), int(lay.status.cpu()[0]), lay)


def assert_layout_equal(ids, e, align):
    c, s, r, f = oracle.layout(ids, e, align)
    gc, gs, gr, gf, lay = gpu_layout(ids, e, align)
    np.testing.assert_array_equal(gc, c)
    np.testing.assert_array_equal(gs, s)
    np.testing.assert_array_equal(gr, r)
    assert gf == f
    return (c, s, r, f), lay


def ulp_diff(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    """Distance in bf16 units in the last place (sign-magnitude aware)."""
    def ordered(b):
        b = b.astype(np.int32)
        return np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF)
    return np.abs(ordered(a_bits) - ordered(b_bits))


# ------------------------------------------------------------------ layout

def test_layout_random_shapes():
    rng = np.random.default_rng(100)
    shapes = [(1, 1, 1), (7, 3, 2), (300, 512, 16), (1000, 64, 16), (4096, 256, 8),
              (513, 17, 16), (8192, 8, 1), (8193, 8, 1), (4097, 2, 2), (2000, 512, 5)]
    for _ in range(30):
        e = int(rng.integers(1, 513))
        k = int(rng.integers(1, min(e, 16) + 1))
        shapes.append((int(rng.integers(1, 1500)), e, k))
    for bs, e, k in shapes:
        for align in (1, 128):
            assert_layout_equal(random_ids(rng, bs, e, k), e, align)


def test_layout_edge_cases():
    rng = np.random.default_rng(101)
    assert_layout_equal(np.zeros((0, 4), np.int32), 16, 128)            # empty batch
    assert_layout_equal(np.zeros((5, 1), np.int32), 1, 128)             # one expert
    e = 16
    assert_layout_equal(np.stack([rng.permutation(e) for _ in range(700)]).astype(np.int32),
                        e, 128)                                         # K = E
    hot = np.array([200, 3, 77, 5, 150, 9, 255, 0], np.int32)
    (c, s, r, f), _ = assert_layout_equal(np.tile(hot, (20000, 1)), 256, 128)  # one hot set
    assert c[hot].min() == 20000
    # at / around the one-workgroup limit (2048 pairs), the per-workgroup
    # tile of the multi-workgroup path (2048 pairs), and ragged tails
    for n in (511, 512, 513, 2047, 2048, 2049, 4095, 4096, 4097, 8193, 12289):
        assert_layout_equal(random_ids(rng, n, 64, 1), 64, 128)


def test_layout_invalid_and_repeated_ids():
    """Out-of-range and repeated ids, with K dividing the 64-lane wave (repeats
    found in the ranking's lane masks) and not (found from the chunk's ids
    staged in LDS), in one-workgroup and multi-workgroup layouts."""
    rng = np.random.default_rng(102)
    for bs, e, k in [(50, 8, 3), (3000, 100, 6), (64, 16, 1), (700, 64, 8), (5000, 256, 8),
                     (300, 32, 16), (9000, 16, 2), (2000, 64, 4), (40000, 512, 16)]:
        ids = random_ids(rng, bs, e, k)
        bad = rng.random(ids.shape) < 0.05
        ids[bad] = rng.choice([-1, e, e + 7, -1000], size=bad.sum())
        (c, s, r, f), _ = assert_layout_equal(ids, e, 128)
        assert f & oracle.FLAG_ID_RANGE
        ids2 = random_ids(rng, bs, e, k)
        ids2[::7, -1] = ids2[::7, 0]
        if k > 2:
            ids2[3::11, 1] = ids2[3::11, 0]  # three copies of one expert in some tokens
            ids2[3::11, 2] = ids2[3::11, 0]
        (c, s, r, f), _ = assert_layout_equal(ids2, e, 128)
        assert f == (oracle.FLAG_DUP_ID if k > 1 else 0)


def test_layout_is_deterministic():
    w = workloads.WORKLOADS["large"]
    ids = workloads.routing(w.bs, w.experts, w.topk, w.routing, w.alpha, w.seed)
    ref = None
    moe = moe_mod()
    d = dev(ids)
    for _ in range(20):
        lay = moe.moe_dispatch_layout(d, w.experts, 128)
        cur = torch.cat([lay.expert_counts, lay.ep_send_counts, lay.expand_idx]).cpu()
        if ref is None:
            ref = cur
        assert torch.equal(cur, ref)


def test_whole_step_is_deterministic():
    """The benchmark's step (moe_dispatch_fused with the read-ahead and the
    cache-resident scatter, then moe_combine) on the skewed workload, 20
    times: layout, dispatched rows and output bit for bit the same."""
    moe = moe_mod()
    w = workloads.WORKLOADS["skewed"]
    cap = oracle.capacity(w.bs, w.topk, w.experts, w.align)
    inp = workloads.make(w, rows_y=cap)
    ids = dev(inp["expert_ids"])
    sc = dev(inp["expert_scales"])
    x, y, sh = inp["x"].to(DEV), inp["y"].to(DEV), inp["shared"].to(DEV)
    ex = torch.empty((cap, w.hidden), dtype=torch.bfloat16, device=DEV)
    ref = None
    for _ in range(20):
        ex.zero_()
        lay, _ = moe.moe_dispatch_fused(x, ids, w.experts, w.align, expand_x=ex,
                                        capacity_rows=cap)
        out = moe.moe_combine(y, ids, lay.expand_idx, lay.ep_send_counts, sc, sh, w.experts)
        torch.cuda.synchronize()
        cur = (torch.cat([lay.expert_counts, lay.ep_send_counts, lay.expand_idx]),
               ex.view(torch.int16).clone(), out.view(torch.int16))
        if ref is None:
            ref = cur
        assert all(torch.equal(a, b) for a, b in zip(cur, ref))


# ------------------------------------------------------------------ dispatch

def run_dispatch_bf16(ids, x_bits, e, align, x_stride=None, out_stride=None, cap=None):
    moe = moe_mod()
    bs, h = x_bits.shape
    c, s, r, _ = oracle.layout(ids, e, align)
    cap = oracle.capacity(bs, ids.shape[1], e, align) if cap is None else cap
    xs = h if x_stride is None else x_stride
    os_ = h if out_stride is None else out_stride
    x_full = np.zeros((bs, xs), np.uint16)
    x_full[:, :h] = x_bits
    xd = bf16_dev(x_full)[:, :h]
    out_full = torch.full((cap, os_), 0, dtype=torch.int16, device=DEV)
    out_full.fill_(np.int16(np.uint16(oracle.SENTINEL_BF16).view(np.int16)))
    out = out_full.view(torch.bfloat16)[:, :h]
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    moe.moe_dispatch(xd, dev(ids), dev(r), dev(s), e, expand_x=out, capacity_rows=cap,
                     status=status)
    torch.cuda.synchronize()
    ref, rflags = oracle.dispatch_bf16(x_bits, ids, r, s, e, cap)
    got = host_bits(out_full.view(torch.bfloat16))
    return got, ref, int(status.cpu()[0]), rflags


@pytest.mark.parametrize("bs,h,e,k,align", [(1, 32, 1, 1, 1), (16, 128, 8, 2, 128),
                                            (37, 1056, 40, 5, 8), (300, 4096, 256, 8, 128),
                                            (129, 7168, 64, 16, 128), (64, 96, 3, 3, 1)])
def test_dispatch_bf16_every_element(bs, h, e, k, align):
    rng = np.random.default_rng(bs * 1000 + h)
    ids = random_ids(rng, bs, e, k)
    x = random_bf16(rng, (bs, h))
    got, ref, gflags, rflags = run_dispatch_bf16(ids, x, e, align)
    assert gflags == rflags == 0
    np.testing.assert_array_equal(got[:, :h], ref)  # padding rows keep the sentinel on both


def test_dispatch_bf16_strided_rows():
    rng = np.random.default_rng(5)
    ids = random_ids(rng, 100, 32, 4)
    x = random_bf16(rng, (100, 512))
    got, ref, _, _ = run_dispatch_bf16(ids, x, 32, 128, x_stride=512 + 64, out_stride=512 + 8)
    np.testing.assert_array_equal(got[:, :512], ref)
    assert np.all(got[:, 512:] == oracle.SENTINEL_BF16)  # stride gap untouched


def test_dispatch_guard_keeps_writes_in_bounds():
    """Capacity one row short of the padded total: the pair landing on the
    missing row is skipped and flagged, and the canary rows after the buffer
    are untouched."""
    moe = moe_mod()
    rng = np.random.default_rng(6)
    e, k, bs, h = 4, 2, 40, 64
    ids = random_ids(rng, bs, e, k)
    c, s, r, _ = oracle.layout(ids, e, 1)
    cap = int(s[-1]) - 1
    canary = 8
    buf = torch.full((cap + canary, h), 0x1234, dtype=torch.int16, device=DEV)
    out = buf.view(torch.bfloat16)[:cap]
    x = random_bf16(rng, (bs, h))
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    moe.moe_dispatch(bf16_dev(x), dev(ids), dev(r), dev(s), e, expand_x=out, capacity_rows=cap,
                     status=status)
    y = torch.zeros((cap, h), dtype=torch.bfloat16, device=DEV)
    ycomb = moe.moe_combine(y, dev(ids), dev(r), dev(s),
                            dev(np.ones((bs, k), np.float32)), None, e, status=status)
    torch.cuda.synchronize()
    assert int(status.cpu()[0]) == oracle.FLAG_GUARD
    assert torch.all(buf[cap:] == 0x1234)
    ref, rflags = oracle.dispatch_bf16(x, ids, r, s, e, cap)
    assert rflags == oracle.FLAG_GUARD
    got = host_bits(out)
    written = ref != oracle.SENTINEL_BF16
    np.testing.assert_array_equal(got[written], ref[written])
    assert ycomb.shape == (bs, h)


def run_dispatch_fp8(ids, x_bits, e, align):
    moe = moe_mod()
    bs, h = x_bits.shape
    c, s, r, _ = oracle.layout(ids, e, align)
    cap = oracle.capacity(bs, ids.shape[1], e, align)
    codes = torch.full((cap, h), oracle.SENTINEL_FP8, dtype=torch.uint8, device=DEV)
    scales = torch.full((cap, h // 128), oracle.SENTINEL_SCALE, dtype=torch.float32, device=DEV)
    moe.moe_dispatch(bf16_dev(x_bits), dev(ids), dev(r), dev(s), e, out_dtype="fp8",
                     expand_x=codes, quant_scales=scales, capacity_rows=cap)
    torch.cuda.synchronize()
    rc, rs, _ = oracle.dispatch_fp8(x_bits, ids, r, s, e, cap)
    return codes.cpu().numpy(), scales.cpu().numpy(), rc, rs


@pytest.mark.parametrize("bs,h,e,k", [(1, 128, 1, 1), (16, 128, 8, 2), (50, 1024, 32, 4),
                                      (200, 7168, 256, 8), (33, 384, 16, 16)])
def test_dispatch_fp8_every_element(bs, h, e, k):
    rng = np.random.default_rng(bs + h)
    ids = random_ids(rng, bs, e, k)
    x = random_bf16(rng, (bs, h))
    x[0, :128] = 0                 # an all-zero block
    x[-1, -128:] = 0x8000          # a block of negative zeros
    gc, gs, rc, rs = run_dispatch_fp8(ids, x, e, 128)
    np.testing.assert_array_equal(gc, rc)
    np.testing.assert_array_equal(gs.view(np.uint32), rs.view(np.uint32))


@pytest.mark.parametrize("bs,h,e,k", [(4096, 4096, 256, 8),   # 32 MiB of rows: read ahead
                                       (4095, 4096, 256, 8),   # just below: scattered from HBM
                                       (8192, 7168, 64, 2),    # 112 MiB of rows, K = 2
                                       (17554, 7168, 64, 2),   # just under 240 MiB: read ahead
                                       (17555, 7168, 64, 2)])  # just over: scattered from HBM
def test_dispatch_with_rows_read_ahead(bs, h, e, k):
    """moe_dispatch to bf16 on contiguous rows of 32 to 240 MB reads them
    ahead in a launch of its own, then scatters in its cache-resident shape:
    the whole buffer against the oracle's, padding untouched; a strided copy
    of the same rows (no read-ahead) and the e4m3 output (never read ahead)
    at the same sizes give the oracle's buffers too."""
    rng = np.random.default_rng(bs + h + k)
    ids = random_ids(rng, bs, e, k)
    x = random_bf16(rng, (bs, h))
    got, ref, gf, rf = run_dispatch_bf16(ids, x, e, 128)
    np.testing.assert_array_equal(got, ref)
    assert gf == rf == 0
    got2, ref2, _, _ = run_dispatch_bf16(ids, x, e, 128, x_stride=h + 64)
    np.testing.assert_array_equal(got2, ref2)
    del got, ref, got2, ref2
    gc, gs, rc, rs = run_dispatch_fp8(ids, x, e, 128)
    np.testing.assert_array_equal(gc, rc)
    np.testing.assert_array_equal(gs.view(np.uint32), rs.view(np.uint32))


def test_fp8_codes_for_every_bf16_value():
    """Every finite bf16 value v with |v| <= 448 quantised in a block whose
    amax is exactly 448 (scale 1: the code is e4m3(v), ties included) and in
    blocks with scales that are not powers of two."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = oracle.bf16_bits_to_f32(bits)
    keep = np.isfinite(vals) & (np.abs(vals) <= 448)
    pool = bits[keep]
    rows = []
    for amax in (448.0, 300.0, 1.0, 3.0e-3):
        amax_bits = oracle.f32_to_bf16_bits(np.array([amax], np.float32))[0]
        av = oracle.bf16_bits_to_f32(np.array([amax_bits]))[0]
        cand = pool[np.abs(oracle.bf16_bits_to_f32(pool)) <= av]
        n_blocks = -(-cand.size // 127)
        padded = np.concatenate([cand, np.zeros(n_blocks * 127 - cand.size, np.uint16)])
        blocks = np.concatenate([np.full((n_blocks, 1), amax_bits, np.uint16),
                                 padded.reshape(n_blocks, 127)], axis=1)
        rows.append(blocks.reshape(-1, 1024) if blocks.size % 1024 == 0 else
                    np.concatenate([blocks.ravel(), np.zeros((-blocks.size) % 1024,
                                                             np.uint16)]).reshape(-1, 1024))
    x = np.concatenate(rows)
    bs = x.shape[0]
    ids = np.zeros((bs, 1), np.int32)
    gc, gs, rc, rs = run_dispatch_fp8(ids, x, 1, 1)
    np.testing.assert_array_equal(gs.view(np.uint32), rs.view(np.uint32))
    np.testing.assert_array_equal(gc, rc)


# ------------------------------------------------------------------ combine

def run_combine(ids, y_bits, scales, shared_bits, e, align, idx_override=None, y_stride=None):
    moe = moe_mod()
    c, s, r, _ = oracle.layout(ids, e, align)
    if idx_override is not None:
        r = idx_override
    cap, h = y_bits.shape
    ys = h if y_stride is None else y_stride
    y_full = np.zeros((cap, ys), np.uint16)
    y_full[:, :h] = y_bits
    yd = bf16_dev(y_full)[:, :h]
    sh = None if shared_bits is None else bf16_dev(shared_bits)
    out = moe.moe_combine(yd, dev(ids), dev(r), dev(s), dev(scales), sh, e)
    torch.cuda.synchronize()
    ref, _ = oracle.combine(y_bits, ids, r, s, scales, shared_bits, e)
    return host_bits(out), ref


@pytest.mark.parametrize("bs,h,e,k,shared", [(1, 32, 1, 1, False), (16, 128, 8, 2, False),
                                             (77, 1056, 40, 5, True), (300, 4096, 256, 8, True),
                                             (65, 7168, 64, 16, True), (50, 7168, 512, 8, False)])
def test_combine_every_element(bs, h, e, k, shared):
    rng = np.random.default_rng(bs * 7 + k)
    ids = random_ids(rng, bs, e, k)
    cap = oracle.capacity(bs, k, e, 128)
    y = random_bf16(rng, (cap, h))
    sc = workloads.scales(bs, k, seed=bs)
    sh = random_bf16(rng, (bs, h)) if shared else None
    got, ref = run_combine(ids, y, sc, sh, e, 128)
    assert ulp_diff(got, ref).max() <= 1
    np.testing.assert_array_equal(got, ref)


def test_combine_strided_y_and_skipped_pairs():
    rng = np.random.default_rng(8)
    bs, h, e, k = 120, 512, 16, 4
    ids = random_ids(rng, bs, e, k)
    c, s, r, _ = oracle.layout(ids, e, 128)
    r = r.copy()
    r[::5] = -1                             # pairs dropped by the caller
    cap = oracle.capacity(bs, k, e, 128)
    y = random_bf16(rng, (cap, h))
    sc = workloads.scales(bs, k, seed=3)
    got, ref = run_combine(ids, y, sc, random_bf16(rng, (bs, h)), e, 128, idx_override=r,
                           y_stride=h + 24)
    np.testing.assert_array_equal(got, ref)


def test_identity_round_trip_on_gpu():
    """layout -> dispatch -> combine with y = dispatched rows, scales summing
    to 1 and no shared row returns x bit for bit."""
    moe = moe_mod()
    rng = np.random.default_rng(9)
    bs, h, e, k = 1000, 2048, 64, 8
    ids = random_ids(rng, bs, e, k)
    x = random_bf16(rng, (bs, h))
    xd = bf16_dev(x)
    lay = moe.moe_dispatch_layout(dev(ids), e, 128)
    ex = moe.moe_dispatch(xd, dev(ids), lay.expand_idx, lay.ep_send_counts, e)
    out = moe.moe_combine(ex, dev(ids), lay.expand_idx, lay.ep_send_counts,
                          dev(workloads.scales(bs, k, seed=1)), None, e)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(oracle.bf16_bits_to_f32(host_bits(out)),
                                  oracle.bf16_bits_to_f32(x))
    assert int(lay.status.cpu()[0]) == 0


# ------------------------------------------------------------------ full-size workloads

def fp8_metrics_dev(codes, scales, x, slots, tok):
    """Max relative error (floor 2^-6 * s) and min row / global cosine of the
    dequantised rows against x, in float64 on the device."""
    q = codes[slots].view(torch.float8_e4m3fn).to(torch.float64)
    s = scales[slots].to(torch.float64).repeat_interleave(128, dim=1)
    deq = q * s
    xv = x[tok].to(torch.float64)
    denom = torch.maximum(xv.abs(), s * 2.0 ** -6)
    rel = torch.where(denom > 0, (deq - xv).abs() / torch.where(denom > 0, denom, 1), 0)
    num = (deq * xv).sum(1)
    den = torch.sqrt((deq * deq).sum(1) * (xv * xv).sum(1))
    cos_rows = torch.where(den > 0, num / torch.where(den > 0, den, 1), 1)
    cos_all = (deq * xv).sum() / torch.sqrt((deq * deq).sum() * (xv * xv).sum())
    return float(rel.max()), float(cos_rows.min()), float(cos_all)


@pytest.mark.parametrize("name", ["tiny", "decode", "skewed", "fp8", "large"])
def test_workload_full_size(name):
    moe = moe_mod()
    w = workloads.WORKLOADS[name]
    print(f"[workload {name}] bs={w.bs} H={w.hidden} E={w.experts} K={w.topk}", flush=True)
    cap = moe.moe_dispatch_capacity(w.bs, w.topk, w.experts, w.align)
    assert cap == oracle.capacity(w.bs, w.topk, w.experts, w.align)
    inp = workloads.make(w, rows_y=cap)
    ids = inp["expert_ids"]
    sc = inp["expert_scales"]

    # layout: every element
    (c, s, r, f), lay = assert_layout_equal(ids, w.experts, w.align)
    assert f == 0
    ids_d = dev(ids)
    x_d = inp["x"].to(DEV)
    slots = torch.from_numpy(s[ids.ravel()].astype(np.int64) + r).to(DEV)
    tok = torch.arange(w.bs, device=DEV).repeat_interleave(w.topk)

    # dispatch: the separate call and moe_dispatch_fused (the call the
    # benchmark times: one launch for decode sizes; else the layout launches
    # that read the rows ahead, then the scatter in its cache-resident or its
    # full-occupancy shape), each into sentinel-filled buffers, so that every
    # padding row must come back untouched
    def sentinel_rows():
        if w.fp8:
            return (torch.full((cap, w.hidden), oracle.SENTINEL_FP8, dtype=torch.uint8,
                               device=DEV),
                    torch.full((cap, w.hidden // 128), oracle.SENTINEL_SCALE,
                               dtype=torch.float32, device=DEV))
        return (torch.full((cap, w.hidden), oracle.SENTINEL_BF16, dtype=torch.int16,
                           device=DEV).view(torch.bfloat16), None)

    kind = "fp8" if w.fp8 else "bf16"
    ex, qs = sentinel_rows()
    moe.moe_dispatch(x_d, ids_d, lay.expand_idx, lay.ep_send_counts, w.experts, out_dtype=kind,
                     capacity_rows=cap, expand_x=ex, quant_scales=qs, check=True)
    fx, fqs = sentinel_rows()
    fused = moe.moe_dispatch_fused(x_d, ids_d, w.experts, w.align, capacity_rows=cap,
                                   out_dtype=kind, expand_x=fx, quant_scales=fqs, check=True)
    torch.cuda.synchronize()
    for a, b in zip(lay, fused[0]):
        assert torch.equal(a, b)
    if w.fp8:
        # every code and scale of the whole buffer, against the oracle's
        # quantisation of each token (padding rows: the sentinels)
        codes_ref, qs_ref, fl = oracle.dispatch_fp8(workloads.bits(inp["x"]), ids, r, s,
                                                    w.experts, cap)
        assert fl == 0
        for what, codes, scales in (("dispatch", ex, qs), ("fused", fx, fqs)):
            np.testing.assert_array_equal(codes.cpu().numpy(), codes_ref, err_msg=what)
            np.testing.assert_array_equal(scales.cpu().numpy().view(np.uint32),
                                          qs_ref.view(np.uint32), err_msg=what)
        sv = slots.view(w.bs, w.topk)
        rel, cmin, call = fp8_metrics_dev(fx, fqs, x_d, sv[:, 0], torch.arange(w.bs, device=DEV))
        print(f"[workload {name}] fp8 max rel {rel:.6f} min row cos {cmin:.6f} "
              f"cos {call:.6f}", flush=True)
        assert rel <= 0.07 and cmin >= 0.999 and call >= 0.999
        del codes_ref, qs_ref
    else:
        # every dispatched row equals its token's row, bit for bit, and every
        # other row still holds the sentinel
        pad = torch.ones(cap, dtype=torch.bool, device=DEV)
        pad[slots] = False
        for what, rows in (("dispatch", ex), ("fused", fx)):
            assert torch.equal(rows[slots].view(torch.int16), x_d[tok].view(torch.int16)), what
            assert bool((rows.view(torch.int16)[pad] == oracle.SENTINEL_BF16).all()), what
        del pad
    del fused, fx, fqs

    # combine: every token against the oracle (at the large workload this
    # includes every token with a row past 2^31 bytes into y)
    if w.identity_experts:
        y_d = ex
        y_bits = oracle.dispatch_bf16(workloads.bits(inp["x"]), ids, r, s, w.experts, cap)[0]
    else:
        y_d = inp["y"].to(DEV)
        y_bits = workloads.bits(inp["y"])
    row_bytes = 2 * w.hidden
    far = int((torch.from_numpy(s[ids.ravel()].astype(np.int64) + r) * row_bytes
               >= 2 ** 31).view(w.bs, w.topk).any(1).sum())
    print(f"[workload {name}] tokens with a row past 2^31 bytes: {far}", flush=True)
    sh = inp["shared"]
    sh_d = None if sh is None else sh.to(DEV)
    out = moe.moe_combine(y_d, ids_d, lay.expand_idx, lay.ep_send_counts, dev(sc), sh_d,
                          w.experts, check=True)
    torch.cuda.synchronize()
    got = host_bits(out)
    ref, fl = oracle.combine(y_bits, ids, r, s, sc, None if sh is None else workloads.bits(sh),
                             w.experts)
    assert fl == 0
    np.testing.assert_array_equal(got, ref)
    if w.identity_experts:
        np.testing.assert_array_equal(oracle.bf16_bits_to_f32(got),
                                      oracle.bf16_bits_to_f32(workloads.bits(inp["x"])))


# ------------------------------------------------------------------ e4m3 combine

def run_combine_fp8(ids, codes, qs, scales, shared_bits, e, align):
    moe = moe_mod()
    c, s, r, _ = oracle.layout(ids, e, align)
    sh = None if shared_bits is None else bf16_dev(shared_bits)
    out = moe.moe_combine_fp8(dev(codes), dev(qs), dev(ids), dev(r), dev(s), dev(scales), sh, e)
    torch.cuda.synchronize()
    ref, _ = oracle.combine_fp8(codes, qs, ids, r, s, scales, shared_bits, e)
    return host_bits(out), ref


def test_combine_fp8_every_code():
    """One-hot weights over rows holding each of the 256 codes, under a scale
    that is not a power of two: exercises the hardware e4m3 decode of every
    code (NaN codes included) against the oracle's decoder."""
    hidden, e = 256, 256
    codes = np.repeat(np.arange(256, dtype=np.uint8)[:, None], hidden, 1)
    qs = np.tile(np.array([[0.37, 3.0e-3]], np.float32), (256, 1))
    ids = np.arange(256, dtype=np.int32).reshape(256, 1)
    got, ref = run_combine_fp8(ids, codes, qs, np.ones((256, 1), np.float32), None, e, 1)
    gf, rf = oracle.bf16_bits_to_f32(got), oracle.bf16_bits_to_f32(ref)
    nan = np.isnan(rf)
    assert np.array_equal(np.isnan(gf), nan)
    np.testing.assert_array_equal(got[~nan], ref[~nan])


@pytest.mark.parametrize("bs,h,e,k,shared", [(1, 128, 1, 1, False), (16, 128, 8, 2, False),
                                             (77, 1152, 40, 5, True), (300, 4096, 256, 8, True),
                                             (65, 7168, 64, 16, True)])
def test_combine_fp8_every_element(bs, h, e, k, shared):
    rng = np.random.default_rng(bs * 11 + k)
    ids = random_ids(rng, bs, e, k)
    cap = oracle.capacity(bs, k, e, 128)
    codes_t, qs_t = workloads.e4m3_rows(cap, h, seed=bs)
    codes, qs = codes_t.numpy(), qs_t.numpy()
    sc = workloads.scales(bs, k, seed=bs)
    sh = random_bf16(rng, (bs, h)) if shared else None
    got, ref = run_combine_fp8(ids, codes, qs, sc, sh, e, 128)
    assert ulp_diff(got, ref).max() <= 1
    np.testing.assert_array_equal(got, ref)


def test_fp8_round_trip_on_gpu():
    """e4m3 dispatch -> e4m3 combine with identity experts: matches the
    oracle's own round trip bit for bit."""
    moe = moe_mod()
    w = workloads.WORKLOADS["fp8"]
    inp = workloads.make(w)
    ids, sc = inp["expert_ids"], inp["expert_scales"]
    ids_d = dev(ids)
    lay = moe.moe_dispatch_layout(ids_d, w.experts, w.align)
    codes, qs = moe.moe_dispatch(inp["x"].to(DEV), ids_d, lay.expand_idx, lay.ep_send_counts,
                                 w.experts, out_dtype="fp8")
    out = moe.moe_combine_fp8(codes, qs, ids_d, lay.expand_idx, lay.ep_send_counts, dev(sc),
                              None, w.experts)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    sample = np.unique(rng.integers(0, w.bs, 48))
    c, s, r, _ = oracle.layout(ids, w.experts, w.align)
    cap = oracle.capacity(w.bs, w.topk, w.experts, w.align)
    x_bits = workloads.bits(inp["x"])
    # the oracle's e4m3 rows for the sampled tokens only, at their own slots
    sub_ids = ids[sample]
    sub_r = r.reshape(w.bs, w.topk)[sample].ravel()
    rc, rq, _ = oracle.dispatch_fp8(x_bits[sample], sub_ids, sub_r, s, w.experts, cap)
    ref, _ = oracle.combine_fp8(rc, rq, sub_ids, sub_r, s, sc[sample], None, w.experts)
    np.testing.assert_array_equal(host_bits(out[torch.from_numpy(sample).to(DEV)]), ref)


# ------------------------------------------------------------------ replica-aware layout

def random_replica_table(rng, e, max_rep):
    reps = rng.integers(1, max_rep + 1, e)
    off = np.concatenate([[0], np.cumsum(reps)]).astype(np.int32)
    thr = np.empty(off[-1], np.uint32)
    for x in range(e):
        w = rng.random(reps[x]) + 0.05
        c = np.cumsum(w / w.sum())
        t = np.minimum(np.floor(c * 4294967296.0), 4294967295).astype(np.uint64)
        t[-1] = 4294967295
        thr[off[x]:off[x + 1]] = t.astype(np.uint32)
    return off, thr


def assert_replicated_equal(ids, e, off, thr, seed, align):
    moe = moe_mod()
    rep, c, s, r, f = oracle.layout_replicated(ids, e, off, thr, seed, align)
    grep, lay = moe.moe_dispatch_layout_replicated(
        dev(ids), e, dev(off), dev(thr.view(np.int32)), seed, align)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(grep.cpu().numpy(), rep)
    np.testing.assert_array_equal(lay.expert_counts.cpu().numpy(), c)
    np.testing.assert_array_equal(lay.ep_send_counts.cpu().numpy(), s)
    np.testing.assert_array_equal(lay.expand_idx.cpu().numpy(), r)
    assert int(lay.status.cpu()[0]) == f
    return rep, s, r, lay, grep


@pytest.mark.parametrize("bs,e,k,max_rep,seed", [(1, 1, 1, 1, 0), (64, 8, 2, 3, 5),
                                                 (700, 64, 8, 4, 11), (4096, 256, 8, 2, 2 ** 40 + 3),
                                                 (5000, 100, 6, 5, 77)])
def test_replicated_layout_matches_oracle(bs, e, k, max_rep, seed):
    rng = np.random.default_rng(bs + e)
    off, thr = random_replica_table(rng, e, max_rep)
    if off[-1] > 512:
        pytest.skip("more than 512 replicas")
    ids = random_ids(rng, bs, e, k)
    for align in (1, 128):
        assert_replicated_equal(ids, e, off, thr, seed, align)


@pytest.mark.parametrize("bs,k", [(3000, 4),    # several workgroups, K divides the wave
                                  (3000, 3),    # several workgroups, ids staged for repeats
                                  (200, 8),     # one workgroup, K divides the wave
                                  (300, 5)])    # one workgroup, ids staged
def test_replicated_layout_flags(bs, k):
    """Out-of-range logical ids, logical experts repeated within a token
    (neighbouring and first-to-last lanes), and an expert whose replicas
    take almost no draw: everything, flags included, as the oracle."""
    rng = np.random.default_rng(3 + k)
    e = 16
    off, thr = random_replica_table(rng, e, 3)
    ids = random_ids(rng, bs, e, k)
    ids[::11, 0] = e + 3                     # out-of-range logical ids
    ids[::13, 2 % k] = ids[::13, 1 % k]      # repeated experts, neighbouring lanes
    ids[5::17, k - 1] = ids[5::17, 0]        # and the token's first and last lanes
    thr = thr.copy()
    thr[off[5]:off[6]] = 0                   # expert 5 can only map when u == 0
    rep, s, r, lay, grep = assert_replicated_equal(ids, e, off, thr, 9, 128)
    f = int(lay.status.cpu()[0])
    assert f & oracle.FLAG_ID_RANGE and f & oracle.FLAG_DUP_ID and f & oracle.FLAG_REPLICA


def test_replicated_pipeline_round_trip():
    """Skewed routing with the 16 hottest experts split into 4 replicas:
    dispatch and combine over the replicas with identity experts return x."""
    moe = moe_mod()
    w = workloads.WORKLOADS["skewed"]
    ids = workloads.routing(w.bs, w.experts, w.topk, w.routing, w.alpha, w.seed)
    hot = workloads.popularity(w.experts, w.routing, w.seed)[:16]
    off, thr = workloads.replica_plan(w.experts, hot, 4)
    p = int(off[-1])
    rep, s, r, lay, grep = assert_replicated_equal(ids, w.experts, off, thr, 1234, 128)
    c_plain = oracle.layout(ids, w.experts, 128)[0]
    # counts gathered per replica add back up to the logical counts
    c_rep = lay.expert_counts.cpu().numpy()
    np.testing.assert_array_equal(np.add.reduceat(c_rep, off[:-1]), c_plain)
    x = workloads.bf16_rows(w.bs, w.hidden, w.seed).to(DEV)
    ex = moe.moe_dispatch(x, grep, lay.expand_idx, lay.ep_send_counts, p)
    out = moe.moe_combine(ex, grep, lay.expand_idx, lay.ep_send_counts,
                          dev(workloads.scales(w.bs, w.topk, w.seed)), None, p)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), x.view(torch.int16))


@pytest.mark.parametrize("bs,h,e,k,max_rep,dtype", [
    (100, 256, 16, 4, 3, "bf16"),      # one layout launch (<= 2048 pairs)
    (700, 512, 64, 8, 4, "bf16"),      # two launches, rows read ahead, cache-resident scatter
    (1200, 1056, 40, 6, 2, "bf16"),    # odd K, ragged row chunks
    (600, 512, 32, 8, 3, "fp8"),
    (2048, 7168, 128, 8, 2, "bf16"),   # prefill row width
])
def test_fused_replicated_matches_oracle(bs, h, e, k, max_rep, dtype):
    """moe_dispatch_fused_replicated equals the oracle's replica-aware layout
    and the oracle's dispatch over replica ids (bf16 rows bit for bit; e4m3
    codes and scales bit for bit), padding rows untouched."""
    moe = moe_mod()
    rng = np.random.default_rng(bs * 3 + k)
    off, thr = random_replica_table(rng, e, max_rep)
    p = int(off[-1])
    assert p <= 512
    ids = random_ids(rng, bs, e, k)
    x_bits = oracle.f32_to_bf16_bits(rng.standard_normal((bs, h)).astype(np.float32))
    seed = 1000 + bs
    rep, c, s, r, f = oracle.layout_replicated(ids, e, off, thr, seed, 128)
    cap = oracle.capacity(bs, k, p, 128)
    if dtype == "bf16":
        buf = torch.full((cap, h), oracle.SENTINEL_BF16, dtype=torch.int16,
                         device=DEV).view(torch.bfloat16)
        grep, lay, ex = moe.moe_dispatch_fused_replicated(
            bf16_dev(x_bits), dev(ids), e, dev(off), dev(thr.view(np.int32)), seed, 128,
            expand_x=buf, capacity_rows=cap)
    else:
        grep, lay, ex, qs = moe.moe_dispatch_fused_replicated(
            bf16_dev(x_bits), dev(ids), e, dev(off), dev(thr.view(np.int32)), seed, 128,
            capacity_rows=cap, out_dtype="fp8")
    torch.cuda.synchronize()
    np.testing.assert_array_equal(grep.cpu().numpy(), rep)
    np.testing.assert_array_equal(lay.expert_counts.cpu().numpy(), c)
    np.testing.assert_array_equal(lay.ep_send_counts.cpu().numpy(), s)
    np.testing.assert_array_equal(lay.expand_idx.cpu().numpy(), r)
    if dtype == "bf16":
        ref_x, f2 = oracle.dispatch_bf16(x_bits, rep, r, s, p, cap)
        assert int(lay.status.cpu()[0]) == (f | f2)
        np.testing.assert_array_equal(host_bits(ex), ref_x)
    else:
        codes_ref, qs_ref, f2 = oracle.dispatch_fp8(x_bits, rep, r, s, p, cap)
        assert int(lay.status.cpu()[0]) == (f | f2)
        slots = (s[rep.ravel()] + r)[rep.ravel() >= 0]
        np.testing.assert_array_equal(ex.cpu().numpy()[slots], codes_ref[slots])
        np.testing.assert_array_equal(qs.cpu().numpy()[slots].view(np.uint32),
                                      qs_ref[slots].view(np.uint32))


# ------------------------------------------------------------------ rank-partitioned layout

@pytest.mark.parametrize("bs,e,k,ws", [(1, 1, 1, 1), (300, 64, 8, 8), (4096, 256, 8, 8),
                                       (5000, 512, 8, 64), (777, 96, 6, 12)])
def test_layout_ep_matches_oracle(bs, e, k, ws):
    moe = moe_mod()
    rng = np.random.default_rng(bs + ws)
    ids = random_ids(rng, bs, e, k)
    for align in (1, 128):
        c, s, ranks, r, f = oracle.layout_ep(ids, e, ws, align)
        lay, granks = moe.moe_dispatch_layout_ep(dev(ids), e, ws, align)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(lay.expert_counts.cpu().numpy(), c)
        np.testing.assert_array_equal(lay.ep_send_counts.cpu().numpy(), s)
        np.testing.assert_array_equal(lay.expand_idx.cpu().numpy(), r)
        np.testing.assert_array_equal(granks.cpu().numpy(), ranks)
        assert int(lay.status.cpu()[0]) == f


# ------------------------------------------------------------ maximum sizes

def test_maximum_dimensions():
    """H = 65536 (the library's largest row), E = 512 experts and K = 16 per
    token at once, through layout, bf16 and e4m3 dispatch, both combines and
    the fused entry point, every element against the oracle (align 1 keeps
    the buffers small)."""
    rng = np.random.default_rng(65536)
    bs, h, e, k, align = 3, 65536, 512, 16, 1
    ids = random_ids(rng, bs, e, k)
    x = random_bf16(rng, (bs, h))
    x[1, 128:256] = 0                       # an all-zero e4m3 block
    (c, s, r, f), _ = assert_layout_equal(ids, e, align)
    cap = oracle.capacity(bs, k, e, align)
    got, ref, gflags, rflags = run_dispatch_bf16(ids, x, e, align)
    assert gflags == rflags == 0
    np.testing.assert_array_equal(got, ref)
    gc, gs, rc, rs = run_dispatch_fp8(ids, x, e, align)
    np.testing.assert_array_equal(gc, rc)
    np.testing.assert_array_equal(gs.view(np.uint32), rs.view(np.uint32))
    y = random_bf16(rng, (cap, h))
    sc = workloads.scales(bs, k, seed=7)
    sh = random_bf16(rng, (bs, h))
    got, ref = run_combine(ids, y, sc, sh, e, align)
    np.testing.assert_array_equal(got, ref)
    got, ref = run_combine_fp8(ids, rc, rs, sc, sh, e, align)
    np.testing.assert_array_equal(got, ref)
    moe = moe_mod()
    lay, ex = moe.moe_dispatch_fused(bf16_dev(x), dev(ids), e, align, capacity_rows=cap)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(lay.expand_idx.cpu().numpy(), r)
    assert cap == bs * k                    # align 1: every row is a real row
    np.testing.assert_array_equal(host_bits(ex), oracle.dispatch_bf16(x, ids, r, s, e, cap)[0])


def test_token_rows_beyond_2gib():
    """150,000 tokens of H = 7168: x, the shared rows and the combine's
    output are 2.15 GB each, so the last tokens' offsets pass 2^31 bytes.
    Through moe_dispatch_fused (bf16: the first 128 MB read ahead and the
    scatter's shape for rows from HBM; e4m3) and moe_combine (identity
    experts, unit weights, x as the shared rows): the layout and the whole
    bf16 buffer against the oracle, and the e4m3 rows and combined tokens
    of the first 1000 and the last 3000 tokens (the oracle's e4m3 and
    combine passes over all 150,000 take most of a minute).  Every row
    carries its token index in two channels (normal bf16 values), so a
    truncated offset reads a row that differs."""
    moe = moe_mod()
    rng = np.random.default_rng(31)
    bs, h, e, k, align = 150_000, 7168, 8, 1, 128
    assert (bs - 3000) * h * 2 < 2**31 < bs * h * 2
    x = np.tile(random_bf16(rng, (4096, h)), ((bs + 4095) // 4096, 1))[:bs]
    tok = np.arange(bs, dtype=np.uint32)
    x[:, 0] = (0x2000 | (tok & 0x1FFF)).astype(np.uint16)
    x[:, 1] = (0x2000 | ((tok >> 13) & 0x1FFF)).astype(np.uint16)
    ids = random_ids(rng, bs, e, k)
    c, s, r, f = oracle.layout(ids, e, align)
    assert f == 0
    cap = oracle.capacity(bs, k, e, align)
    xd, idd = bf16_dev(x), dev(ids)
    sentinel = int(np.uint16(oracle.SENTINEL_BF16).view(np.int16))
    sub = np.concatenate([np.arange(1000), np.arange(bs - 3000, bs)])
    sub_slots = (s[ids[sub]] + r.reshape(bs, k)[sub]).reshape(-1)

    ex = torch.full((cap, h), sentinel, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    lay, _ = moe.moe_dispatch_fused(xd, idd, e, align, expand_x=ex, capacity_rows=cap)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(lay.expert_counts.cpu().numpy(), c)
    np.testing.assert_array_equal(lay.ep_send_counts.cpu().numpy(), s)
    np.testing.assert_array_equal(lay.expand_idx.cpu().numpy(), r)
    assert int(lay.status.cpu()[0]) == 0
    y = host_bits(ex)
    ref, rf = oracle.dispatch_bf16(x, ids, r, s, e, cap)
    assert rf == 0
    np.testing.assert_array_equal(y, ref)
    del ref

    sc = np.ones((bs, k), np.float32)
    out = moe.moe_combine(ex, idd, lay.expand_idx, lay.ep_send_counts, dev(sc), xd, e)
    torch.cuda.synchronize()
    got = out[torch.from_numpy(sub).to(DEV)]
    ref, rf = oracle.combine(y, ids[sub], r.reshape(bs, k)[sub].reshape(-1), s, sc[sub],
                             x[sub], e)
    assert rf == 0
    np.testing.assert_array_equal(host_bits(got), ref)
    del out, got, ref, y, ex

    codes = torch.full((cap, h), oracle.SENTINEL_FP8, dtype=torch.uint8, device=DEV)
    qs = torch.full((cap, h // 128), oracle.SENTINEL_SCALE, dtype=torch.float32, device=DEV)
    moe.moe_dispatch_fused(xd, idd, e, align, capacity_rows=cap, out_dtype="fp8",
                           expand_x=codes, quant_scales=qs)
    torch.cuda.synchronize()
    rc, rs, rf = oracle.dispatch_fp8(x[sub], ids[sub], r.reshape(bs, k)[sub].reshape(-1), s, e,
                                     cap)
    assert rf == 0
    rows = torch.from_numpy(sub_slots).to(DEV)
    np.testing.assert_array_equal(codes[rows].cpu().numpy(), rc[sub_slots])
    np.testing.assert_array_equal(qs[rows].cpu().numpy().view(np.uint32),
                                  rs[sub_slots].view(np.uint32))


def test_maximum_row_two_launch_fused():
    """moe_dispatch_fused above 2048 pairs at the largest row (H = 65536,
    E = 512, K = 16): the layout launch reads the 26 MB of rows ahead and the
    scatter runs in its cache-resident shape (128 chunks of 64 threads per
    row); every element against the oracle."""
    moe = moe_mod()
    rng = np.random.default_rng(200)
    bs, h, e, k, align = 200, 65536, 512, 16, 1
    ids = random_ids(rng, bs, e, k)
    x = random_bf16(rng, (bs, h))
    c, s, r, f = oracle.layout(ids, e, align)
    cap = oracle.capacity(bs, k, e, align)
    lay, ex = moe.moe_dispatch_fused(bf16_dev(x), dev(ids), e, align, capacity_rows=cap)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(lay.expert_counts.cpu().numpy(), c)
    np.testing.assert_array_equal(lay.ep_send_counts.cpu().numpy(), s)
    np.testing.assert_array_equal(lay.expand_idx.cpu().numpy(), r)
    assert int(lay.status.cpu()[0]) == f == 0
    assert cap == bs * k                    # align 1: every row is a real row
    np.testing.assert_array_equal(host_bits(ex), oracle.dispatch_bf16(x, ids, r, s, e, cap)[0])


def test_layout_many_workgroups_every_expert_count():
    """Tens to 256 ranking workgroups with E from 1 to 512, so the last
    workgroup's column scan runs with 512 down to 1 threads per column, on
    4-column (16-byte) and single columns (E not a multiple of 4), with its
    rows kept in registers between the passes or read again."""
    rng = np.random.default_rng(103)
    for bs, e, k in [(200000, 1, 1), (60000, 3, 2), (100000, 8, 2), (30000, 100, 8),
                     (40000, 300, 4), (30000, 512, 16), (100000, 511, 3), (60000, 37, 5)]:
        assert_layout_equal(random_ids(rng, bs, e, k), e, 128)


def rotated_ids(rng, bs, e, k):
    """Distinct ids per row at sizes where a per-row argsort is too slow:
    (h_t + j) mod E for a uniform start h_t (k <= E)."""
    h = rng.integers(0, e, size=bs, dtype=np.int32)
    ids = np.empty((bs, k), np.int32)
    for j in range(k):
        np.add(h, j, out=ids[:, j])
        np.remainder(ids[:, j], e, out=ids[:, j])
    return ids


def test_layout_multi_chunk_workgroups():
    """Batches beyond 256 workgroups of 2048 pairs: each ranking workgroup
    walks several chunks of whole tokens (K not dividing 2048 as well), and
    the scan over the workgroups' histograms runs once."""
    rng = np.random.default_rng(104)
    for bs, e, k in [(100000, 37, 7), (80000, 512, 16), (600000, 1, 1), (200001, 200, 3),
                     (140000, 64, 5)]:
        (c, s, r, f), _ = assert_layout_equal(rotated_ids(rng, bs, e, k), e, 128)
        assert int(c.sum()) == bs * k and f == 0


@pytest.mark.parametrize("pairs,e,k", [(4 << 20, 256, 8), (16 << 20, 512, 8)])
def test_layout_millions_of_pairs(pairs, e, k):
    """The work-efficient scan at 4M and 16M pairs, bit-exact."""
    rng = np.random.default_rng(105 + pairs % 97)
    ids = rotated_ids(rng, pairs // k, e, k)
    ids[::1013] = np.arange(k, dtype=np.int32)[::-1]  # a recurring token on the same experts
    (c, s, r, f), _ = assert_layout_equal(ids, e, 128)
    assert int(c.sum()) == pairs and f == 0


def test_layout_largest_batch():
    """The largest batch the argument rules admit at E = 512, K = 16,
    align = 128: 67,104,807 tokens (1,073,676,912 pairs), whose padded
    capacity is exactly 2^30 rows.  Layout only (the ids need no token rows)."""
    moe = moe_mod()
    e, k, align = 512, 16, 128
    bs = 67104807
    assert moe.moe_dispatch_capacity(bs, k, e, align) == 1 << 30
    with pytest.raises(moe.MoeError):
        moe.moe_dispatch_capacity(bs + 1, k, e, align)
    rng = np.random.default_rng(106)
    ids = rotated_ids(rng, bs, e, k)
    (c, s, r, f), _ = assert_layout_equal(ids, e, align)
    assert int(c.sum()) == bs * k and f == 0


def sentinel_layout(e, n):
    """Layout outputs filled with -7, so that an output a call fails to
    write cannot pass by holding an earlier call's values."""
    moe = moe_mod()
    return moe.Layout(*(torch.full((m,), -7, dtype=torch.int32, device=DEV)
                        for m in (e, e + 1, n, 1)))


def test_workspace_reused_across_shapes():
    """One caller workspace, zero-filled once, serves a run of layout and
    fused calls of changing shapes (multi-workgroup and one-launch), each
    bit-exact against the oracle; the arrival counter, the workspace's first
    word, is zero after every call."""
    moe = moe_mod()
    rng = np.random.default_rng(107)
    shapes = [(3000, 256, 8), (700, 64, 6), (100, 64, 8), (4096, 256, 8), (20000, 512, 16),
              (600, 17, 3), (70000, 1, 1), (4096, 256, 8)]
    size = max(moe.moe_dispatch_layout_workspace_size(bs, k, e) for bs, e, k in shapes)
    ws = torch.zeros(size, dtype=torch.uint8, device=DEV)
    h = 128
    for i, (bs, e, k) in enumerate(shapes):
        ids = random_ids(rng, bs, e, k)
        c, s, r, f = oracle.layout(ids, e, 128)
        lay = moe.moe_dispatch_layout(dev(ids), e, 128, out=sentinel_layout(e, bs * k),
                                      workspace=ws)
        x = random_bf16(rng, (bs, h))
        cap = oracle.capacity(bs, k, e, 128)
        rows = torch.full((cap, h), oracle.SENTINEL_BF16, dtype=torch.int16,
                          device=DEV).view(torch.bfloat16)
        fused, _ = moe.moe_dispatch_fused(bf16_dev(x), dev(ids), e, 128,
                                          out=sentinel_layout(e, bs * k), capacity_rows=cap,
                                          expand_x=rows, workspace=ws)
        torch.cuda.synchronize()
        for got in (lay, fused):
            np.testing.assert_array_equal(got.expert_counts.cpu().numpy(), c, err_msg=str(i))
            np.testing.assert_array_equal(got.ep_send_counts.cpu().numpy(), s, err_msg=str(i))
            np.testing.assert_array_equal(got.expand_idx.cpu().numpy(), r, err_msg=str(i))
            assert int(got.status.cpu()[0]) == f
        np.testing.assert_array_equal(host_bits(rows),
                                      oracle.dispatch_bf16(x, ids, r, s, e, cap)[0])
        assert int(ws[:4].view(torch.int32)[0]) == 0
