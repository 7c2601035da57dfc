"""Pins for the oracle's replica-aware layout (TEMPO summary, section 2,
system integration: probabilistic replica dispatch with count gathering in
one kernel).

* the generator against the published SplitMix64 reference draws
  (tests/golden/splitmix64_seed0.txt);
* the replica choice against a second formulation (numpy searchsorted over
  each expert's threshold slice) and the layout over replicas against the
  stable-argsort formulation;
* closed forms (one replica per expert reduces to the plain layout; a
  threshold of 2^32-1 on the first replica always picks it);
* choice frequencies against the thresholds (chi-square);
* malformed tables are flagged, never mapped.
"""

import os

import numpy as np
import pytest

import oracle
from test_oracle_layout import layout_by_argsort

HERE = os.path.dirname(os.path.abspath(__file__))
GAMMA = np.uint64(0x9E3779B97F4A7C15)


def test_splitmix64_reference_draws():
    rows = [l.split() for l in open(os.path.join(HERE, "golden", "splitmix64_seed0.txt"))
            if l.strip() and not l.startswith("#")]
    assert len(rows) == 3
    for i, v in rows:
        assert oracle.splitmix64(0, int(i)) == int(v, 16)


def random_table(rng, e, max_rep):
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


def choose_by_searchsorted(ids, off, thr, seed):
    """Second formulation: u from the per-pair draws, replica = the expert's
    slice position found by numpy.searchsorted (first threshold >= u)."""
    flat = ids.ravel()
    u = np.array([oracle.splitmix64(seed, i) >> 32 for i in range(flat.size)], np.uint64)
    out = np.empty(flat.size, np.int64)
    for i, e in enumerate(flat):
        sl = thr[off[e]:off[e + 1]].astype(np.uint64)
        pos = int(np.searchsorted(sl, u[i], side="left"))
        out[i] = off[e] + pos if pos < sl.size else -1
    return out.reshape(ids.shape)


@pytest.mark.parametrize("seed", [0, 12345, 2 ** 63 + 7])
def test_choice_and_layout_against_second_formulation(seed):
    rng = np.random.default_rng(seed % 1000)
    e, k, bs = 24, 4, 300
    off, thr = random_table(rng, e, 4)
    p = int(off[-1])
    ids = np.argsort(rng.random((bs, e)), axis=1)[:, :k].astype(np.int32)
    rep, counts, send, idx, flags = oracle.layout_replicated(ids, e, off, thr, seed, 128)
    assert flags == 0
    np.testing.assert_array_equal(rep, choose_by_searchsorted(ids, off, thr, seed))
    c2, s2, r2 = layout_by_argsort(rep, p, 128)
    np.testing.assert_array_equal(counts, c2)
    np.testing.assert_array_equal(send, s2)
    np.testing.assert_array_equal(idx, r2)
    # every chosen replica belongs to its logical expert
    assert np.all((rep >= off[ids]) & (rep < off[ids + 1]))


def test_one_replica_per_expert_is_the_plain_layout():
    rng = np.random.default_rng(4)
    e, k, bs = 64, 8, 500
    ids = np.argsort(rng.random((bs, e)), axis=1)[:, :k].astype(np.int32)
    off = np.arange(e + 1, dtype=np.int32)
    thr = np.full(e, 0xFFFFFFFF, np.uint32)
    rep, counts, send, idx, flags = oracle.layout_replicated(ids, e, off, thr, 99, 128)
    c, s, r, f = oracle.layout(ids, e, 128)
    np.testing.assert_array_equal(rep, ids)
    np.testing.assert_array_equal(counts, c)
    np.testing.assert_array_equal(send, s)
    np.testing.assert_array_equal(idx, r)
    assert flags == f == 0


def test_full_threshold_on_first_replica_always_wins():
    ids = np.array([[0, 1], [1, 0], [0, 1]], np.int32)
    off = np.array([0, 3, 5], np.int32)
    thr = np.array([0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF], np.uint32)
    rep, *_ = oracle.layout_replicated(ids, 2, off, thr, 7, 1)
    np.testing.assert_array_equal(rep, [[0, 3], [3, 0], [0, 3]])


def test_choice_frequencies_follow_thresholds():
    e, k, bs = 2, 1, 200000
    probs = np.array([0.5, 0.3, 0.2])
    c = np.cumsum(probs)
    thr = np.minimum(np.floor(c * 4294967296.0), 4294967295).astype(np.uint64)
    thr[-1] = 4294967295
    off = np.array([0, 3, 4], np.int32)
    thr_all = np.concatenate([thr, [4294967295]]).astype(np.uint32)
    ids = np.zeros((bs, 1), np.int32)
    rep, counts, *_ = oracle.layout_replicated(ids, e, off, thr_all, 2024, 1)
    obs = counts[:3].astype(np.float64)
    exp = probs * bs
    chi2 = ((obs - exp) ** 2 / exp).sum()
    assert chi2 < 13.8  # 2 degrees of freedom, p = 0.001


def test_malformed_tables_are_flagged():
    ids = np.array([[0, 1]], np.int32)
    off = np.array([0, 0, 2], np.int32)          # expert 0 has no replica
    thr = np.array([0xFFFFFFFF, 0xFFFFFFFF], np.uint32)
    rep, counts, send, idx, flags = oracle.layout_replicated(ids, 2, off, thr, 1, 1)
    assert flags & oracle.FLAG_REPLICA
    assert rep[0, 0] == -1 and idx[0] == -1 and rep[0, 1] == 0
    thr0 = np.array([0], np.uint32)              # threshold 0: only u == 0 maps
    rep, _, _, _, flags = oracle.layout_replicated(np.array([[0]], np.int32), 1,
                                                  np.array([0, 1], np.int32), thr0, 5, 1)
    assert rep[0, 0] == -1 and flags & oracle.FLAG_REPLICA
