"""The pages' argument rules (tests/golden/argument_rules.txt, each line with
its source) against the oracle's argument checks."""

import os

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def load_rules():
    rules = {}
    with open(os.path.join(HERE, "golden", "argument_rules.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, value, source = line.split(None, 2)
            rules[name] = (value, source)
    return rules


def test_rules_file_has_sources():
    rules = load_rules()
    assert len(rules) >= 10
    for name, (value, source) in rules.items():
        assert source.strip(), name


def test_expert_num_range():
    r = load_rules()
    lo, hi = int(r["expert_num_min"][0]), int(r["expert_num_max"][0])
    assert oracle.check_layout_args(4, 1, lo, 128) == oracle.OK
    assert oracle.check_layout_args(4, 1, hi, 128) == oracle.OK
    assert oracle.check_layout_args(4, 1, lo - 1, 128) == oracle.ERR_INVALID_ARG
    assert oracle.check_layout_args(4, 1, hi + 1, 128) == oracle.ERR_INVALID_ARG


def test_topk_range():
    r = load_rules()
    kmax = int(r["topk_max"][0])
    assert oracle.check_layout_args(4, kmax, 64, 128) == oracle.OK
    assert oracle.check_layout_args(4, kmax + 1, 64, 128) == oracle.ERR_INVALID_ARG
    assert oracle.check_layout_args(4, 0, 64, 128) == oracle.ERR_INVALID_ARG
    assert oracle.check_layout_args(4, 5, 4, 128) == oracle.ERR_INVALID_ARG  # K > E


def test_hidden_rules():
    r = load_rules()
    m = int(r["hidden_multiple"][0])
    assert oracle.check_row_args(m, 0) == oracle.OK
    assert oracle.check_row_args(m + 16, 0) == oracle.ERR_INVALID_ARG
    # the product cap H <= 7168 is not adopted
    assert "not-adopted" in r["hidden_max"][1]
    assert oracle.check_row_args(int(r["hidden_max"][0]) * 2, 0) == oracle.OK


def test_batch_cap_not_adopted():
    r = load_rules()
    assert "not-adopted" in r["bs_max"][1]
    assert oracle.check_layout_args(int(r["bs_max"][0]) * 32, 8, 256, 128) == oracle.OK


def test_tile_rows_default():
    r = load_rules()
    assert int(r["segment_tile_rows"][0]) == 128
    assert oracle.check_layout_args(16, 2, 8, int(r["segment_tile_rows"][0])) == oracle.OK
