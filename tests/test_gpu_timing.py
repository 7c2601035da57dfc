"""Kernel timing by bound events (moe_time_next_launches, include/moe_probe.h):
each launch takes one event pair in launch order, the outputs do not change,
the pairs' kernel times fit inside events recorded around the whole step,
and a call that fails launches nothing and leaves its pairs bound."""

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu


def random_ids(rng, bs, e, k):
    return np.argsort(rng.random((bs, e)), axis=1)[:, :k].astype(np.int32)


def new_pairs(n):
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(n)]
    for a, z in pairs:
        a.record()
        z.record()
    return pairs


@pytest.mark.parametrize("bs,expect_launches", [(600, 3), (100, 2)])
def test_bound_events_time_each_launch(bs, expect_launches):
    """Ranking launch (with its scan) + scatter + combine (600 tokens, 4800
    pairs) and the single fused launch + combine (100 tokens, 800 pairs)."""
    import combine_moe_dispatch_layout_amd as moe
    h, e, k = 1024, 64, 8
    rng = np.random.default_rng(bs)
    ids_np = random_ids(rng, bs, e, k)
    x = torch.from_numpy(
        oracle.f32_to_bf16_bits(rng.standard_normal((bs, h)).astype(np.float32)).view(np.int16)
    ).view(torch.bfloat16).cuda()
    sc = torch.from_numpy(rng.random((bs, k)).astype(np.float32)).cuda()
    ids = torch.from_numpy(ids_np).cuda()

    def step():
        lay, ex = moe.moe_dispatch_fused(x, ids, e)
        return lay, moe.moe_combine(ex, ids, lay.expand_idx, lay.ep_send_counts, sc, None, e)

    lay0, out0 = step()
    torch.cuda.synchronize()

    pairs = new_pairs(16)
    outer = new_pairs(1)[0]
    outer[0].record()
    moe.moe_time_next_launches(pairs)
    lay1, out1 = step()
    outer[1].record()
    used = 16 - moe.moe_time_unused_launches()
    moe.moe_time_next_launches([])
    assert moe.moe_time_unused_launches() == 0
    torch.cuda.synchronize()
    assert used == expect_launches
    times = [a.elapsed_time(z) for a, z in pairs[:used]]
    whole = outer[0].elapsed_time(outer[1])
    assert all(t > 0 for t in times), times
    assert sum(times) <= whole * 1.001 + 1e-3, (times, whole)
    # bound pairs follow launch order: each kernel starts after the last ended
    for (a0, z0), (a1, _) in zip(pairs[:used - 1], pairs[1:used]):
        assert z0.elapsed_time(a1) >= -1e-3
    np.testing.assert_array_equal(lay1.expand_idx.cpu().numpy(), lay0.expand_idx.cpu().numpy())
    assert torch.equal(out1.view(torch.int16), out0.view(torch.int16))
    c, s, r, f = oracle.layout(ids_np, e, 128)
    np.testing.assert_array_equal(lay1.expand_idx.cpu().numpy(), r)


def test_failed_call_leaves_pairs_bound():
    import combine_moe_dispatch_layout_amd as moe
    pairs = new_pairs(2)
    moe.moe_time_next_launches(pairs)
    ids = torch.zeros((4, 2), dtype=torch.int32, device="cuda")
    with pytest.raises(moe.MoeError):
        moe.moe_dispatch_layout(ids, 1)      # k = 2 > num_experts = 1: rejected
    assert moe.moe_time_unused_launches() == 2
    moe.moe_time_next_launches([])
    assert moe.moe_time_unused_launches() == 0


def test_bindings_are_per_host_thread():
    """Pairs bound on one host thread are taken only by that thread's
    launches: a second thread launching meanwhile leaves them bound."""
    import threading

    import combine_moe_dispatch_layout_amd as moe
    rng = np.random.default_rng(21)
    ids = torch.from_numpy(random_ids(rng, 300, 64, 8)).cuda()
    pairs = new_pairs(4)
    torch.cuda.synchronize()
    moe.moe_time_next_launches(pairs)
    seen = {}

    def other():
        try:
            seen["before"] = moe.moe_time_unused_launches()   # nothing bound on this thread
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                moe.moe_dispatch_layout(ids, 64)
            stream.synchronize()
            seen["after"] = moe.moe_time_unused_launches()
        except Exception as err:  # reported below
            seen["error"] = err

    t = threading.Thread(target=other)
    t.start()
    t.join(timeout=60)
    assert "error" not in seen, seen.get("error")
    assert seen == {"before": 0, "after": 0}
    assert moe.moe_time_unused_launches() == 4       # this thread's pairs untouched
    moe.moe_dispatch_layout(ids, 64)                 # 2400 pairs: two layout launches
    assert moe.moe_time_unused_launches() == 2
    moe.moe_time_next_launches([])
    torch.cuda.synchronize()
    for a, z in pairs[:2]:
        assert a.elapsed_time(z) > 0

