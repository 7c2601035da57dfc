"""Pins for the oracle's layout (counts, padded prefix, stable ranks).

The oracle is checked against things other than itself:
* brute force over every routing of tiny problems, compared with a second,
  independent formulation built on numpy's stable argsort and bincount;
* invariants and closed forms that the definition fixes (counts sum to BS*K,
  128-aligned offsets, slot bijection, K = E, all tokens on the same experts);
* the pages' id rules (range [0, E), no repeats within a row) as flags.
"""

import itertools

import numpy as np
import pytest

import oracle
import workloads


def layout_by_argsort(ids: np.ndarray, num_experts: int, align: int):
    """Second formulation: the unpadded expert-contiguous order is the stable
    argsort of the flattened ids; a pair's rank is its position in that order
    minus the position where its expert's run starts."""
    flat = ids.ravel()
    counts = np.bincount(flat, minlength=num_experts).astype(np.int64)
    padded = -(-counts // align) * align
    send = np.concatenate([[0], np.cumsum(padded)])
    order = np.argsort(flat, kind="stable")
    run_start = np.concatenate([[0], np.cumsum(counts)])
    rank = np.empty(flat.size, dtype=np.int64)
    rank[order] = np.arange(flat.size) - run_start[flat[order]]
    return counts, send, rank


def all_routings(bs, num_experts, k):
    rows = list(itertools.permutations(range(num_experts), k))
    for combo in itertools.product(rows, repeat=bs):
        yield np.array(combo, dtype=np.int32).reshape(bs, k)


@pytest.mark.parametrize("bs,num_experts,k", [(1, 1, 1), (2, 2, 2), (3, 3, 1), (3, 4, 2),
                                              (2, 4, 3), (3, 2, 1)])
@pytest.mark.parametrize("align", [1, 2, 4, 128])
def test_bruteforce_every_routing(bs, num_experts, k, align):
    n_cases = 0
    for ids in all_routings(bs, num_experts, k):
        c, s, r, flags = oracle.layout(ids, num_experts, align)
        c2, s2, r2 = layout_by_argsort(ids, num_experts, align)
        assert flags == 0
        np.testing.assert_array_equal(c, c2)
        np.testing.assert_array_equal(s, s2)
        np.testing.assert_array_equal(r, r2)
        n_cases += 1
    assert n_cases > 0


def test_bruteforce_case_count():
    # ordered distinct rows: (E!/(E-K)!)^BS
    assert sum(1 for _ in all_routings(3, 4, 2)) == 12 ** 3


def check_invariants(ids, num_experts, align):
    bs, k = ids.shape
    c, send, r, flags = oracle.layout(ids, num_experts, align)
    assert flags == 0
    assert c.sum() == bs * k
    assert send[0] == 0 and np.all(send % align == 0)
    np.testing.assert_array_equal(np.diff(send), -(-c.astype(np.int64) // align) * align)
    assert send[-1] <= oracle.capacity(bs, k, num_experts, align)
    flat = ids.ravel()
    slot = send[flat].astype(np.int64) + r
    # bijection from pairs onto the real rows  U_e [send[e], send[e] + c[e])
    assert np.unique(slot).size == slot.size
    assert np.all(r >= 0) and np.all(r < c[flat])
    # within a segment, the token index strictly increases with the slot
    tok = np.repeat(np.arange(bs), k)
    order = np.argsort(slot)
    seg = flat[order]
    same = seg[1:] == seg[:-1]
    assert np.all(tok[order][1:][same] > tok[order][:-1][same])
    return c, send, r


@pytest.mark.parametrize("name", ["tiny", "decode", "skewed", "fp8", "large"])
def test_invariants_on_workloads(name):
    w = workloads.WORKLOADS[name]
    ids = workloads.routing(w.bs, w.experts, w.topk, w.routing, w.alpha, w.seed)
    c, send, r = check_invariants(ids, w.experts, w.align)
    c2, send2, r2 = layout_by_argsort(ids, w.experts, w.align)
    np.testing.assert_array_equal(c, c2)
    np.testing.assert_array_equal(send, send2)
    np.testing.assert_array_equal(r, r2)


@pytest.mark.parametrize("align", [1, 128])
def test_random_shapes_against_argsort(align):
    rng = np.random.default_rng(7)
    for _ in range(60):
        num_experts = int(rng.integers(1, 513))
        k = int(rng.integers(1, min(num_experts, 16) + 1))
        bs = int(rng.integers(1, 300))
        ids = np.argsort(rng.random((bs, num_experts)), axis=1)[:, :k].astype(np.int32)
        check_invariants(ids, num_experts, align)
        c, s, r, _ = oracle.layout(ids, num_experts, align)
        c2, s2, r2 = layout_by_argsort(ids, num_experts, align)
        np.testing.assert_array_equal(r, r2)
        np.testing.assert_array_equal(s, s2)


def test_closed_form_k_equals_e():
    bs, e = 37, 6
    rng = np.random.default_rng(1)
    ids = np.stack([rng.permutation(e) for _ in range(bs)]).astype(np.int32)
    c, send, r, _ = oracle.layout(ids, e, 128)
    assert np.all(c == bs)
    np.testing.assert_array_equal(send, np.arange(e + 1) * 128)
    np.testing.assert_array_equal(r.reshape(bs, e), np.repeat(np.arange(bs)[:, None], e, 1))


def test_closed_form_all_tokens_same_experts():
    bs, e, k = 1000, 256, 8
    hot = np.array([200, 3, 77, 5, 150, 9, 255, 0], dtype=np.int32)
    ids = np.tile(hot, (bs, 1))
    c, send, r, _ = oracle.layout(ids, e, 128)
    expect = np.zeros(e, dtype=np.int64)
    expect[hot] = bs
    np.testing.assert_array_equal(c, expect)
    assert send[-1] == k * 1024  # ceil(1000/128)*128 = 1024 per hot expert
    np.testing.assert_array_equal(r.reshape(bs, k), np.repeat(np.arange(bs)[:, None], k, 1))


def test_empty_batch():
    c, send, r, flags = oracle.layout(np.zeros((0, 4), dtype=np.int32), 16, 128)
    assert c.sum() == 0 and np.all(send == 0) and r.size == 0 and flags == 0


def test_out_of_range_ids_are_flagged_and_dropped():
    ids = np.array([[0, 5], [-1, 1], [1, 0]], dtype=np.int32)
    c, send, r, flags = oracle.layout(ids, 4, 1)
    assert flags == oracle.FLAG_ID_RANGE
    np.testing.assert_array_equal(c, [2, 2, 0, 0])
    np.testing.assert_array_equal(r, [0, -1, -1, 0, 1, 1])
    np.testing.assert_array_equal(send, [0, 2, 4, 4, 4])


def test_duplicate_ids_are_flagged_and_laid_out_stably():
    ids = np.array([[2, 2], [2, 0]], dtype=np.int32)
    c, send, r, flags = oracle.layout(ids, 3, 1)
    assert flags == oracle.FLAG_DUP_ID
    np.testing.assert_array_equal(c, [1, 0, 3])
    np.testing.assert_array_equal(r, [0, 1, 2, 0])


@pytest.mark.parametrize("bs,k,e,align", [(4, 1, 0, 128), (4, 1, 513, 128), (4, 0, 8, 128),
                                          (4, 9, 8, 128), (4, 17, 64, 128), (4, 2, 8, 3),
                                          (4, 2, 8, 2048), (-1, 2, 8, 128), (4, 2, 8, 0)])
def test_argument_rules_reject(bs, k, e, align):
    assert oracle.check_layout_args(bs, k, e, align) == oracle.ERR_INVALID_ARG


@pytest.mark.parametrize("bs,k,e,align", [(1, 1, 1, 1), (0, 8, 256, 128), (16384, 8, 512, 128),
                                          (4, 16, 16, 1024), (512, 8, 512, 128)])
def test_argument_rules_accept(bs, k, e, align):
    assert oracle.check_layout_args(bs, k, e, align) == oracle.OK


def test_capacity_is_tight():
    # the bound is reached when every expert holds one token more than a
    # multiple of the alignment
    e, k, align = 8, 2, 4
    ids = np.arange(e, dtype=np.int32).reshape(e // k, k)  # c_e = 1 for every expert
    c, send, _, _ = oracle.layout(ids, e, align)
    assert np.all(c == 1)
    assert send[-1] == oracle.capacity(e // k, k, e, align) == 32
    # and never exceeded on random routings
    rng = np.random.default_rng(3)
    for _ in range(200):
        num_experts = int(rng.integers(1, 40))
        kk = int(rng.integers(1, min(num_experts, 16) + 1))
        bs = int(rng.integers(0, 50))
        a = int(2 ** rng.integers(0, 8))
        ids = np.argsort(rng.random((bs, num_experts)), axis=1)[:, :kk].astype(np.int32)
        _, s, _, _ = oracle.layout(ids.reshape(bs, kk), num_experts, a)
        assert s[-1] <= oracle.capacity(bs, kk, num_experts, a)


def test_equal_out_of_range_ids_are_not_a_repeated_expert():
    # "repeats" concerns experts, i.e. ids in [0, E); two equal invalid ids in
    # a row only raise the range flag
    ids = np.array([[-1, -1], [7, 7], [0, 1]], dtype=np.int32)
    c, send, r, flags = oracle.layout(ids, 4, 1)
    assert flags == oracle.FLAG_ID_RANGE
    np.testing.assert_array_equal(r, [-1, -1, -1, -1, 0, 0])


def test_random_bad_and_repeated_ids_against_argsort():
    """Out-of-range ids are dropped (rank -1, not counted) and repeats are
    ranked in row-major order like distinct pairs: the argsort formulation
    restricted to the valid pairs gives the same layout, and the flags are
    set exactly when such ids occur."""
    rng = np.random.default_rng(17)
    for trial in range(120):
        num_experts = int(rng.integers(1, 65))
        k = int(rng.integers(1, min(num_experts, 16) + 1))
        bs = int(rng.integers(0, 120))
        ids = rng.integers(0, num_experts, size=(bs, k)).astype(np.int32)   # repeats likely
        bad = rng.random(ids.shape) < (0.1 if trial % 2 else 0.0)
        ids[bad] = rng.choice([-1, num_experts, num_experts + 3, -50], size=int(bad.sum()))
        c, s, r, f = oracle.layout(ids, num_experts, 128)
        flat = ids.ravel()
        valid = (flat >= 0) & (flat < num_experts)
        c2, s2, r2 = layout_by_argsort(flat[valid].reshape(-1, 1) if valid.any()
                                       else np.zeros((0, 1), np.int32), num_experts, 128)
        np.testing.assert_array_equal(c, c2)
        np.testing.assert_array_equal(s, s2)
        np.testing.assert_array_equal(r[valid], r2)
        assert np.all(r[~valid] == -1)
        rows_repeat = any(len(set(v for v in row if 0 <= v < num_experts)) <
                          sum(1 for v in row if 0 <= v < num_experts) for row in ids)
        assert bool(f & oracle.FLAG_ID_RANGE) == bool((~valid).any())
        assert bool(f & oracle.FLAG_DUP_ID) == rows_repeat
