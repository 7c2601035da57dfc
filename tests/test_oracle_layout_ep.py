"""Pins for the oracle's rank-partitioned layout (combine page: A3-series
ep_send_counts has ep_world_size * local_expert_num entries; experts divide
evenly over the expert ranks)."""

import numpy as np
import pytest

import oracle


def test_rank_segments_hold_exactly_their_experts_pairs():
    rng = np.random.default_rng(0)
    e, k, bs, ws = 64, 6, 800, 8
    ids = np.argsort(rng.random((bs, e)), axis=1)[:, :k].astype(np.int32)
    for align in (1, 128):
        c, s, ranks, idx, f = oracle.layout_ep(ids, e, ws, align)
        L = e // ws
        slot = s[ids.ravel()].astype(np.int64) + idx
        dest = np.searchsorted(ranks, slot, side="right") - 1
        np.testing.assert_array_equal(dest, ids.ravel() // L)   # each pair in its rank's range
        rows = np.diff(ranks)
        padded = -(-c.astype(np.int64) // align) * align
        np.testing.assert_array_equal(rows, padded.reshape(ws, L).sum(1))
        assert ranks[0] == 0 and ranks[-1] == s[-1]


def test_closed_forms():
    rng = np.random.default_rng(1)
    e, k, bs = 16, 2, 100
    ids = np.argsort(rng.random((bs, e)), axis=1)[:, :k].astype(np.int32)
    c, s, ranks, _, _ = oracle.layout_ep(ids, e, 1, 128)
    np.testing.assert_array_equal(ranks, [0, s[-1]])                 # one rank: everything
    c, s, ranks, _, _ = oracle.layout_ep(ids, e, e, 128)
    np.testing.assert_array_equal(ranks, s)                          # one expert per rank
    c0, s0, idx0, _ = oracle.layout(ids, e, 128)
    c, s, ranks, idx, _ = oracle.layout_ep(ids, e, 4, 128)
    np.testing.assert_array_equal(idx, idx0)                         # same ranks and offsets
    np.testing.assert_array_equal(s, s0)


@pytest.mark.parametrize("e,ws", [(16, 3), (16, 0), (8, 16), (16, -2)])
def test_rejects_uneven_or_invalid_world_size(e, ws):
    with pytest.raises(oracle.OracleArgError):
        oracle.layout_ep(np.zeros((2, 1), np.int32), e, ws, 128)
