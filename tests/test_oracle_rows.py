"""The oracle's gated apply and per-row report against hand cases and a
bit-string brute force (TensorRT-Edge-LLM "Guided Decoder": a zero row flag
leaves the row alone; an all-zero in-range mask row admits no token)."""

import math

import numpy as np
import pytest

import oracle
from _golden import build_case, expected_positions, load

DATA = load()
ROWS = DATA["rows_cases"]["cases"]
NEG_INF = {"float32": 0xFF800000, "float16": 0xFC00, "bfloat16": 0xFF80}


@pytest.mark.parametrize("case", ROWS, ids=[c["name"] for c in ROWS])
def test_rows_hand_case(case):
    logits, mask = build_case(case)
    gate = None if case["gate"] is None else np.array(case["gate"], dtype=np.int8)
    got, any_allowed = oracle.apply_rows(logits.copy(), mask, case["dtype"], case["vocab_size"], gate)
    want = logits.copy()
    for r, cols in expected_positions(case).items():
        for c in cols:
            want[r, c] = NEG_INF[case["dtype"]]
    assert np.array_equal(got, want)
    assert any_allowed.tolist() == case["any"]


@pytest.mark.parametrize("seed", range(20))
def test_report_against_bit_strings(seed):
    rng = np.random.default_rng(500 + seed)
    rows = int(rng.integers(1, 6))
    mcols = int(rng.integers(1, 5))
    V = int(rng.integers(0, 32 * mcols + 1))
    dens = float(rng.choice([0.0, 0.002, 0.05, 0.5]))
    bits = rng.random((rows, 32 * mcols)) < dens
    mask = np.packbits(bits, axis=1, bitorder="little").view("<u4").reshape(rows, mcols).view(np.int32)
    gate = (rng.random(rows) < 0.7).astype(np.int8)
    logits = rng.integers(0, 2**16, size=(rows, max(V, 1)), dtype=np.uint64).astype(np.uint16)
    _, rep = oracle.apply_rows(logits.copy(), mask, "float16", V, gate)
    for r in range(rows):
        s = "".join(format(int(w) & 0xFFFFFFFF, "032b")[::-1] for w in mask[r])
        want = (1 if V > 0 else 0) if gate[r] == 0 else (1 if "1" in s[:V] else 0)
        assert rep[r] == want, (r, V, gate[r])
