"""Prepared calls on the GPU: moe.prepare() checks an entry point's call once
and returns a callable that repeats its launch on the same tensors.  Each
prepared call, repeated with new contents in the same input tensors, must
give what the direct call gives (layout and dispatched rows bit for bit,
the combined rows bit for bit): the fused path in its one-launch and
two-launch forms, the separate calls, and the combine."""

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


@pytest.mark.parametrize("bs,h,e,k", [(128, 1024, 64, 8),     # one fused launch
                                      (3000, 1024, 64, 8)])   # layout + scatter launches
def test_prepared_step_equals_direct_calls(bs, h, e, k):
    import combine_moe_dispatch_layout_amd as moe
    rng = np.random.default_rng(bs + h)
    ids = torch.from_numpy(random_ids(rng, bs, e, k)).to(DEV)
    x = to_dev_bf16(random_bf16(rng, (bs, h)))
    sc = torch.from_numpy(rng.random((bs, k)).astype(np.float32)).to(DEV)
    sh = to_dev_bf16(random_bf16(rng, (bs, h)))
    ws = torch.zeros(max(moe.moe_dispatch_layout_workspace_size(bs, k, e), 16),
                     dtype=torch.uint8, device=DEV)
    front = moe.prepare(moe.moe_dispatch_fused, x, ids, e, 128, workspace=ws)
    lay, ex = front.result
    back = moe.prepare(moe.moe_combine, ex, ids, lay.expand_idx, lay.ep_send_counts, sc, sh, e)
    out = back.result
    for rep in range(3):
        # new routing and rows in the same tensors
        ids.copy_(torch.from_numpy(random_ids(rng, bs, e, k)))
        x.copy_(to_dev_bf16(random_bf16(rng, (bs, h))))
        ex.zero_()
        front()
        back()
        torch.cuda.synchronize()
        got = [t.clone() for t in lay] + [ex.view(torch.int16).clone(), out.view(torch.int16).clone()]
        ref_lay, ref_ex = moe.moe_dispatch_fused(x, ids, e, 128)
        ref_out = moe.moe_combine(ref_ex, ids, ref_lay.expand_idx, ref_lay.ep_send_counts, sc, sh, e)
        torch.cuda.synchronize()
        for a, b in zip(got[:4], ref_lay):
            assert torch.equal(a, b), rep
        slots = (ref_lay.ep_send_counts[ids.reshape(-1).long()] + ref_lay.expand_idx).long()
        assert torch.equal(got[4][slots], ref_ex.view(torch.int16)[slots]), rep
        assert torch.equal(got[5], ref_out.view(torch.int16)), rep
        c, s, r, f = oracle.layout(ids.cpu().numpy(), e, 128)
        np.testing.assert_array_equal(got[2].cpu().numpy(), r)


def test_prepared_separate_calls():
    import combine_moe_dispatch_layout_amd as moe
    rng = np.random.default_rng(11)
    bs, h, e, k = 2500, 512, 32, 4
    ids = torch.from_numpy(random_ids(rng, bs, e, k)).to(DEV)
    x = to_dev_bf16(random_bf16(rng, (bs, h)))
    ws = torch.zeros(max(moe.moe_dispatch_layout_workspace_size(bs, k, e), 16),
                     dtype=torch.uint8, device=DEV)
    lay_call = moe.prepare(moe.moe_dispatch_layout, ids, e, 128, workspace=ws)
    lay = lay_call.result
    disp = moe.prepare(moe.moe_dispatch, x, ids, lay.expand_idx, lay.ep_send_counts, e,
                       out_dtype="fp8")
    codes, qs = disp.result
    for rep in range(2):
        ids.copy_(torch.from_numpy(random_ids(rng, bs, e, k)))
        x.copy_(to_dev_bf16(random_bf16(rng, (bs, h))))
        lay_call()
        disp()
        torch.cuda.synchronize()
        ids_h = ids.cpu().numpy()
        c, s, r, f = oracle.layout(ids_h, e, 128)
        np.testing.assert_array_equal(lay.expand_idx.cpu().numpy(), r)
        np.testing.assert_array_equal(lay.ep_send_counts.cpu().numpy(), s)
        x_bits = x.view(torch.int16).cpu().numpy().view(np.uint16)
        cap = codes.shape[0]
        rc, rs, _ = oracle.dispatch_fp8(x_bits, ids_h, r, s, e, cap)
        slots = s[ids_h.ravel()].astype(np.int64) + r
        np.testing.assert_array_equal(codes.cpu().numpy()[slots], rc[slots])
        np.testing.assert_array_equal(qs.cpu().numpy()[slots].view(np.uint32),
                                      rs[slots].view(np.uint32))
