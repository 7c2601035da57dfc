"""The layout -> dispatch -> combine path captured once in a HIP graph
(torch.cuda.CUDAGraph) and replayed on new inputs.

No entry point allocates, synchronises or enqueues a memset when its outputs
and workspace are passed in, so a captured step must reproduce the oracle on
every replay.  Each replay gets fresh seeded routing, weights and rows copied
into the captured buffers, and eager library calls plus a device
synchronisation run between replays.  Combine consumes the dispatched rows
(identity experts), so the replay covers the whole chain; both the one-launch
layout (<= 2048 pairs) and the two-launch layout with its workspace are
captured, through the separate calls and through moe_dispatch_fused.
"""

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu


def random_ids(rng, bs, e, k):
    return np.argsort(rng.random((bs, e)), axis=1)[:, :k].astype(np.int32)


def random_bf16(rng, shape):
    return oracle.f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32))


def to_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)


def bits_of(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def make_inputs(rng, bs, hidden, e, k, with_shared):
    ids = random_ids(rng, bs, e, k)
    logits = rng.standard_normal((bs, k))
    w = np.exp(logits - logits.max(axis=1, keepdims=True))
    scales = (w / w.sum(axis=1, keepdims=True)).astype(np.float32)
    x = random_bf16(rng, (bs, hidden))
    shared = random_bf16(rng, (bs, hidden)) if with_shared else None
    return ids, scales, x, shared


@pytest.mark.parametrize("path", ["separate", "fused"])
@pytest.mark.parametrize("bs,hidden,e,k,with_shared", [
    (40, 256, 16, 4, True),       # one-launch layout (fused: one launch for both)
    (700, 384, 64, 8, False),     # two-launch layout, three ranking workgroups (fused: with
                                  # the rows read ahead and the cache-resident scatter shape)
    (128, 7168, 256, 8, True),    # decode shape
])
def test_captured_step_replays_match_the_oracle(bs, hidden, e, k, with_shared, path):
    import combine_moe_dispatch_layout_amd as moe
    moe.load_library()
    dev = torch.device("cuda", 0)
    cap = moe.moe_dispatch_capacity(bs, k, e, 128)
    rng = np.random.default_rng(900 + bs)

    ids0, sc0, x0, sh0 = make_inputs(rng, bs, hidden, e, k, with_shared)
    ids = torch.from_numpy(ids0).to(dev)
    scales = torch.from_numpy(sc0).to(dev)
    x = to_bf16(x0).to(dev)
    shared = to_bf16(sh0).to(dev) if with_shared else None
    lay = moe.Layout(torch.empty(e, dtype=torch.int32, device=dev),
                     torch.empty(e + 1, dtype=torch.int32, device=dev),
                     torch.empty(bs * k, dtype=torch.int32, device=dev),
                     torch.empty(1, dtype=torch.int32, device=dev))
    ws = torch.zeros(max(moe.moe_dispatch_layout_workspace_size(bs, k, e), 16),
                     dtype=torch.uint8, device=dev)  # zero-filled before its first use
    expand_x = torch.empty((cap, hidden), dtype=torch.bfloat16, device=dev)
    out = torch.empty((bs, hidden), dtype=torch.bfloat16, device=dev)

    def step():
        if path == "fused":
            moe.moe_dispatch_fused(x, ids, e, 128, out=lay, capacity_rows=cap,
                                   expand_x=expand_x, workspace=ws)
        else:
            moe.moe_dispatch_layout(ids, e, 128, out=lay, workspace=ws)
            moe.moe_dispatch(x, ids, lay.expand_idx, lay.ep_send_counts, e, expand_x=expand_x,
                             capacity_rows=cap)
        moe.moe_combine(expand_x, ids, lay.expand_idx, lay.ep_send_counts, scales, shared, e,
                        out=out)

    step()  # eager warm-up before capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    side_ids = torch.from_numpy(random_ids(rng, 3000, 32, 2)).to(dev)
    for replay in range(4):
        ids_np, sc_np, x_np, sh_np = make_inputs(rng, bs, hidden, e, k, with_shared)
        ids.copy_(torch.from_numpy(ids_np))
        scales.copy_(torch.from_numpy(sc_np))
        x.copy_(to_bf16(x_np))
        if with_shared:
            shared.copy_(to_bf16(sh_np))
        graph.replay()
        side = moe.moe_dispatch_layout(side_ids, 32, 128)  # eager work between replays
        torch.cuda.synchronize()
        assert int(side.status.cpu()[0]) == 0

        c, s, r, f = oracle.layout(ids_np, e, 128)
        np.testing.assert_array_equal(lay.expert_counts.cpu().numpy(), c, err_msg=f"replay {replay}")
        np.testing.assert_array_equal(lay.ep_send_counts.cpu().numpy(), s)
        np.testing.assert_array_equal(lay.expand_idx.cpu().numpy(), r)
        assert int(lay.status.cpu()[0]) == f == 0

        ref_x, _ = oracle.dispatch_bf16(x_np, ids_np, r, s, e, cap)
        slots = (s[ids_np.reshape(-1)] + r).reshape(-1)
        got_x = bits_of(expand_x)
        np.testing.assert_array_equal(got_x[slots], ref_x[slots], err_msg=f"replay {replay}")

        ref_out, _ = oracle.combine(ref_x, ids_np, r, s, sc_np, sh_np, e)
        np.testing.assert_array_equal(bits_of(out), ref_out, err_msg=f"replay {replay}")
