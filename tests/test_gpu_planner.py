"""The compensation planner fed by the GPU layout, as it is used: the
per-expert counts that moe_dispatch_layout computes on the device for the
skewed and large workloads go straight into moe_plan_compensation, and the
plan must equal the oracle planner's over the oracle layout's counts, move
for move, with the same loads and bounds, at 8, 16 and 64 ranks (DeepEP
compensation PR, Python section: the 128-aligned compensation planner that
consumes the counts the dispatch gathers)."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle import planner

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    import combine_moe_dispatch_layout_amd as m
    m.load_library()
    assert torch.cuda.is_available()
    return m


@pytest.mark.parametrize("name", ["skewed", "large"])
def test_plan_from_device_counts(moe, name):
    w = workloads.WORKLOADS[name]
    ids = workloads.routing(w.bs, w.experts, w.topk, w.routing, w.alpha, w.seed)
    lay = moe.moe_dispatch_layout(torch.from_numpy(ids).cuda(), w.experts, w.align, check=True)
    device_counts = lay.expert_counts.cpu().numpy()
    ref_counts = oracle.layout(ids, w.experts, w.align)[0]
    np.testing.assert_array_equal(device_counts, ref_counts)
    for ws in (8, 16, 64):
        got = moe.moe_plan_compensation(lay.expert_counts, ws, 8, 10)
        ref = planner.plan(ref_counts, ws, 8, 10)
        assert got["moves"] == [tuple(m) for m in ref["moves"]], (name, ws)
        assert got["loads"] == list(ref["loads"])
        assert (got["before"], got["after"], got["ideal"]) == (
            ref["before"], ref["after"], ref["ideal"])
        assert got["after"] <= got["before"]
        assert all(m[3] % 128 == 0 for m in got["moves"])   # whole 128-row chunks
