"""Oracle against hand-worked cases (tests/golden/hand_cases.json).

Each case's expected masked columns were worked out by hand from one rule the
pages state (the case carries its citation).  Both oracle forms -- the
pure-Python loop and the C loop -- must reproduce every case bit for bit.
"""

import numpy as np
import pytest

import oracle
from _golden import build_case, expected_positions, fill_of, load, parse_value

DATA = load()
CASES = DATA["cases"]
FILL_CASES = DATA["fill_cases"]["cases"]


def golden_fill_bits(case):
    if "fill_bits" in case:
        return int(case["fill_bits"], 16)
    for f in FILL_CASES:
        if f["value"] == case["fill"] and f["dtype"] == case["dtype"]:
            return int(f["bits"], 16)
    raise KeyError(case["name"])


@pytest.mark.parametrize("impl", ["py", "c"])
@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_hand_case(case, impl):
    logits, mask = build_case(case)
    args = dict(vocab_size=case["vocab_size"], indices=case["indices"], fill_value=fill_of(case))
    if impl == "py":
        got = oracle.apply_inplace_py(logits, mask, case["dtype"], **args)
    else:
        got = oracle.apply_inplace(logits.copy(), mask, case["dtype"], **args)
    want = logits.copy()
    fb = golden_fill_bits(case)
    for r, cols in expected_positions(case).items():
        for c in cols:
            want[r, c] = fb
    assert np.array_equal(got, want)


@pytest.mark.parametrize("fc", FILL_CASES, ids=[f"{f['dtype']}:{f['value']}" for f in FILL_CASES])
def test_fill_case(fc):
    assert oracle.fill_bits(parse_value(fc["value"]), fc["dtype"]) == int(fc["bits"], 16)


def test_default_vocab_rule_examples():
    # XGrammar "Bitmask Operations", Notes: Padding
    assert oracle.resolve_vocab_size(50257, 1571) == 50257
    assert oracle.resolve_vocab_size(128256, 4008) == 128256
    assert oracle.resolve_vocab_size(128256, 4008, 128000) == 128000
    assert oracle.resolve_vocab_size(40, 1) == 32
    assert oracle.resolve_vocab_size(20, 2) == 20
    with pytest.raises(ValueError):
        oracle.resolve_vocab_size(40, 1, 33)
    with pytest.raises(ValueError):
        oracle.resolve_vocab_size(20, 2, 21)
    with pytest.raises(ValueError):
        oracle.resolve_vocab_size(20, 2, -1)


def test_row_set_rules():
    # XGrammar "Bitmask Operations", Notes: Indices
    assert oracle.row_set(3, 3) == [0, 1, 2]
    assert oracle.row_set(4, 2, [1]) == [1]
    with pytest.raises(ValueError):
        oracle.row_set(4, 2, [2])      # valid only below both batch sizes
    with pytest.raises(ValueError):
        oracle.row_set(4, 4, [-1])
    with pytest.raises(ValueError):
        oracle.row_set(4, 3)           # without indices every logits row needs a mask row
