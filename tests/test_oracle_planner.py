"""Pins for the oracle of the 128-aligned compensation planner.

The planner is a heuristic, so its oracle is the plain step-by-step reading
(oracle/planner.py); these tests pin that reading to things outside itself:
* invariants the model fixes (rows conserved per expert, moves in whole
  128-row chunks, reported loads equal the loads recomputed from the final
  assignment, makespan never above the start, never below the ideal bound);
* brute force: on tiny instances every 128-aligned split of every expert's
  chunks is enumerated, and the planner is within one chunk plus one
  activation of that optimum;
* closed forms (one hot expert between two ranks splits evenly; balanced
  loads give no move; min_gain above the reachable gain gives a no-op);
* quality on the workloads' per-expert counts (DeepEP PR reports ~99 % of
  the ideal bound).
"""

import itertools

import numpy as np
import pytest

import oracle
import workloads
from oracle import planner

CH = planner.CHUNK


def loads_of(assign, tile, act):
    return [sum(act + tile * (-(-a // CH)) for a in row if a > 0) for row in assign]


def final_assignment(counts, ws, moves):
    e_n = len(counts)
    per = e_n // ws
    assign = [[0] * e_n for _ in range(ws)]
    for e, c in enumerate(counts):
        assign[e // per][e] = c
    for e, src, dst, rows in moves:
        assert rows > 0 and rows % CH == 0
        assert assign[src][e] >= rows
        assign[src][e] -= rows
        assign[dst][e] += rows
    return assign


def check_invariants(counts, ws, tile, act, res):
    assign = final_assignment(counts, ws, res["moves"])
    for e, c in enumerate(counts):
        assert sum(assign[r][e] for r in range(ws)) == c
    assert loads_of(assign, tile, act) == res["loads"]
    assert res["after"] == max(res["loads"]) <= res["before"]
    assert res["after"] >= res["ideal"]


@pytest.mark.parametrize("seed", range(6))
def test_invariants_random(seed):
    rng = np.random.default_rng(seed)
    ws = int(rng.choice([2, 3, 4, 8]))
    e_n = ws * int(rng.integers(1, 9))
    counts = (rng.zipf(1.6, e_n) * rng.integers(10, 200)).clip(0, 20000)
    tile, act = int(rng.integers(1, 20)), int(rng.integers(0, 40))
    res = planner.plan(counts, ws, tile, act)
    check_invariants(counts, ws, tile, act, res)


def brute_force_optimum(counts, ws, tile, act):
    """Every way to hand each expert's whole 128-row chunks to the ranks (the
    remainder stays on the home rank)."""
    e_n = len(counts)
    per = e_n // ws
    choices = []
    for e, c in enumerate(counts):
        m = c // CH
        opts = []
        for split in itertools.product(range(m + 1), repeat=ws):
            if sum(split) != m:
                continue
            rows = [s * CH for s in split]
            rows[e // per] += c - m * CH
            opts.append(rows)
        choices.append(opts)
    best = None
    for combo in itertools.product(*choices):
        loads = [sum(act + tile * (-(-combo[e][r] // CH)) for e in range(e_n)
                     if combo[e][r] > 0) for r in range(ws)]
        best = max(loads) if best is None else min(best, max(loads))
    return best


@pytest.mark.parametrize("counts,ws,tile,act", [
    ([1024, 0], 2, 8, 10), ([512, 384, 0, 128], 2, 8, 10), ([640, 100, 256, 0], 2, 5, 3),
    ([384, 0, 0], 3, 8, 4), ([512, 256, 0, 0, 0, 0], 3, 6, 9), ([300, 700, 50, 0], 2, 7, 2),
])
def test_within_one_chunk_and_activation_of_brute_force(counts, ws, tile, act):
    res = planner.plan(counts, ws, tile, act)
    check_invariants(counts, ws, tile, act, res)
    opt = brute_force_optimum(counts, ws, tile, act)
    assert opt <= res["after"] <= opt + tile + act


def test_one_hot_expert_splits_evenly():
    res = planner.plan([1024, 0, 0, 0], 2, tile=8, activation=10)
    assert res["moves"] == [(0, 0, 1, 512)]
    assert res["loads"] == [42, 42] and res["before"] == 74


def test_balanced_gives_no_move_and_min_gain_gives_no_op():
    assert planner.plan([256, 256, 256, 256], 4, 8, 10)["moves"] == []
    res = planner.plan([1024, 0, 0, 0], 2, 8, 10, min_gain=33)   # reachable gain is 32
    assert res["moves"] == [] and res["after"] == res["before"] == 74
    res = planner.plan([1024, 0, 0, 0], 2, 8, 10, min_gain=32)
    assert res["moves"] and res["after"] == 42


@pytest.mark.parametrize("name,ws", [("skewed", 8), ("large", 8), ("large", 16)])
def test_quality_on_workload_counts(name, ws):
    w = workloads.WORKLOADS[name]
    ids = workloads.routing(w.bs, w.experts, w.topk, w.routing, w.alpha, w.seed)
    counts = oracle.layout(ids, w.experts, 128)[0]
    # TEMPO's flat regime: an expert's floor costs about as much as 1.25
    # tiles (n* ~ 160 tokens against 128-token tiles)
    res = planner.plan(counts, ws, tile=8, activation=10)
    check_invariants(counts, ws, 8, 10, res)
    quality = res["ideal"] / res["after"]
    assert res["after"] < res["before"]
    assert quality >= 0.95, quality
