"""moe_dispatch_fused_noalloc (the layout workspace in the library's static
per-GPU scratch) against moe_dispatch_fused (a caller workspace), through the
C ABI, bit for bit: counts, offsets, ranks, status, every row of the
dispatched buffer (padding rows keep their sentinel) and the e4m3 scales.
Several calls run in a row on the one scratch, the second smaller than the
first, so a call that left the scratch in a wrong state would show; a batch
too large for the scratch is refused before anything is enqueued."""

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def moe():
    import combine_moe_dispatch_layout_amd as m
    m.load_library()
    assert torch.cuda.is_available()
    return m


def routing(rng, bs, e, k):
    return np.argsort(rng.random((bs, e)), axis=1)[:, :k].astype(np.int32)


def token_rows(rng, bs, h):
    bits = oracle.f32_to_bf16_bits(rng.standard_normal((bs, h)).astype(np.float32))
    return torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16)


def sentinel_rows(cap, h, dtype):
    if dtype == "bf16":
        return torch.full((cap, h), oracle.SENTINEL_BF16, dtype=torch.int16,
                          device=DEV).view(torch.bfloat16)
    return torch.full((cap, h), oracle.SENTINEL_FP8, dtype=torch.uint8, device=DEV)


def both_paths(moe, bs, h, e, k, dtype, seed):
    """Runs both entry points on the same inputs into sentinel-filled
    buffers and returns their outputs as host arrays."""
    rng = np.random.default_rng(seed)
    ids = torch.from_numpy(routing(rng, bs, e, k)).to(DEV)
    x = token_rows(rng, bs, h)
    cap = moe.moe_dispatch_capacity(bs, k, e, 128)
    res = []
    for fn in (moe.moe_dispatch_fused, moe.moe_dispatch_fused_noalloc):
        rows = sentinel_rows(cap, h, dtype)
        # outputs pre-filled with -7: an output a call fails to write shows
        lay_out = moe.Layout(*(torch.full((m,), -7, dtype=torch.int32, device=DEV)
                               for m in (e, e + 1, bs * k, 1)))
        scales = (torch.full((cap, h // 128), oracle.SENTINEL_SCALE, dtype=torch.float32,
                             device=DEV) if dtype == "fp8" else None)
        out = fn(x, ids, e, 128, out=lay_out, capacity_rows=cap, out_dtype=dtype,
                 expand_x=rows, quant_scales=scales)
        lay = out[0]
        torch.cuda.synchronize()
        res.append([lay.expert_counts.cpu().numpy(), lay.ep_send_counts.cpu().numpy(),
                    lay.expand_idx.cpu().numpy(), lay.status.cpu().numpy(),
                    rows.view(torch.uint8).cpu().numpy()]
                   + ([scales.cpu().numpy()] if scales is not None else []))
    return res


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_noalloc_matches_fused_on_consecutive_calls(moe, dtype):
    # first a larger batch, then a smaller one on the same scratch, then a
    # decode-sized batch (one launch, no scratch), then larger ones again,
    # with other expert counts
    for i, (bs, h, e, k) in enumerate([(3000, 1024, 256, 8), (700, 512, 64, 6),
                                       (128, 1024, 256, 8), (4096, 512, 256, 8),
                                       (20000, 256, 512, 16), (600, 256, 17, 3)]):
        ref, got = both_paths(moe, bs, h, e, k, dtype, seed=100 + i)
        names = ["expert_counts", "ep_send_counts", "expand_idx", "status", "expand_x",
                 "quant_scales"]
        for name, a, b in zip(names, ref, got):
            np.testing.assert_array_equal(b, a, err_msg=f"call {i} ({bs}x{k}): {name}")
        assert int(ref[3][0]) == 0


def test_noalloc_refuses_a_batch_beyond_its_scratch(moe):
    bs, k, e = 170000, 8, 512
    need = moe.moe_dispatch_layout_workspace_size(bs, k, e)
    assert need > moe.moe_noalloc_scratch_bytes()
    ids = torch.zeros((bs, k), dtype=torch.int32, device=DEV)
    x = torch.zeros((bs, 128), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(moe.MoeError) as err:
        moe.moe_dispatch_fused_noalloc(x, ids, e, 128, capacity_rows=0)
    assert err.value.code == moe.MOE_ERR_SCRATCH
    # the largest batch the scratch always holds: 2^20 pairs at E = 512
    assert moe.moe_dispatch_layout_workspace_size((1 << 20) // 8, 8, 512) <= \
        moe.moe_noalloc_scratch_bytes()
