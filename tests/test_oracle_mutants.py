"""The pins catch plausible mistakes planted in the oracle.

Each mutant below replaces one piece of the (pure-Python) oracle with a
plausibly wrong version; the pins -- the hand cases, the fill cases and a
small bit-string brute force -- must reject every one, and accept the
oracle as it is.  Mutants live only in this process, on the CPU.
"""

import math

import numpy as np
import pytest

import oracle
from _golden import build_case, expected_positions, fill_of, load, parse_value

DATA = load()


def pins_pass() -> bool:
    fills = DATA["fill_cases"]["cases"]
    for f in fills:
        if oracle.fill_bits(parse_value(f["value"]), f["dtype"]) != int(f["bits"], 16):
            return False
    for case in DATA["cases"]:
        if case["cols"] > 2000:
            continue
        logits, mask = build_case(case)
        try:
            got = oracle.apply_inplace_py(logits, mask, case["dtype"], case["vocab_size"],
                                          case["indices"], fill_of(case))
        except (ValueError, IndexError):
            return False
        fb = int(case.get("fill_bits", "0") or "0", 16) if "fill_bits" in case else None
        if fb is None:
            fb = next(int(f["bits"], 16) for f in fills
                      if f["value"] == case["fill"] and f["dtype"] == case["dtype"])
        want = logits.copy()
        for r, cols in expected_positions(case).items():
            for c in cols:
                want[r, c] = fb
        if not np.array_equal(got, want):
            return False
    # bit-string brute force on a few random rows
    rng = np.random.default_rng(3)
    for _ in range(20):
        cols = int(rng.integers(1, 80))
        mask = rng.integers(0, 2**32, size=(2, 3), dtype=np.uint64).astype(np.uint32).view(np.int32)
        logits = rng.integers(0, 2**16, size=(2, cols), dtype=np.uint64).astype(np.uint16)
        fb = 0xFF80
        want = logits.copy()
        for i in range(2):
            s = "".join(format(int(w) & 0xFFFFFFFF, "032b")[::-1] for w in mask[i])
            for j in range(cols):
                if s[j] == "0":
                    want[i, j] = fb
        try:
            got = oracle.apply_inplace_py(logits, mask, "bfloat16")
        except (ValueError, IndexError):
            return False
        if not np.array_equal(got, want):
            return False
    return True


def test_oracle_as_is_passes():
    assert pins_pass()


def _bit_msb_first(bitmask, i, j):
    return (int(bitmask[i][j // 32]) & 0xFFFFFFFF) >> (31 - j % 32) & 1


def _bit_inverted(bitmask, i, j):
    return 1 - ((int(bitmask[i][j // 32]) & 0xFFFFFFFF) >> (j % 32) & 1)


def _bit_word_index_16(bitmask, i, j):
    return (int(bitmask[i][j // 16 if j // 16 < len(bitmask[i]) else -1]) & 0xFFFFFFFF) >> (j % 32) & 1


def _bit_row_zero(bitmask, i, j):
    return (int(bitmask[0][j // 32]) & 0xFFFFFFFF) >> (j % 32) & 1


_orig_resolve = oracle.resolve_vocab_size
_orig_row_set = oracle.row_set
_orig_fill = oracle.fill_bits
_orig_loops = oracle.apply_inplace_loops


def _vocab_max(cols, mask_cols, vocab_size=None):
    return max(cols, 32 * mask_cols) if vocab_size is None else vocab_size


def _vocab_cols_only(cols, mask_cols, vocab_size=None):
    return cols if vocab_size is None else vocab_size


def _vocab_off_by_one(cols, mask_cols, vocab_size=None):
    return _orig_resolve(cols, mask_cols, vocab_size) - (1 if vocab_size is None else 0)


def _rows_ignore_indices(rows, mask_rows, indices=None):
    return _orig_row_set(rows, mask_rows, None if mask_rows >= rows else indices)


def _rows_sorted_positions(rows, mask_rows, indices=None):
    # uses the position in the index list instead of the index itself
    return list(range(len(indices))) if indices is not None else _orig_row_set(rows, mask_rows)


def _decode(bits, dtype):
    if dtype == "float16":
        return float(np.uint16(bits).view(np.float16))
    if dtype == "float32":
        return float(np.uint32(bits).view(np.float32))
    return float(np.uint32(bits << 16).view(np.float32))


def _fill_truncate(value, dtype):
    r = _orig_fill(value, dtype)
    if math.isnan(value) or math.isinf(value):
        return r
    # step one pattern toward zero whenever rounding went away from zero
    return r - 1 if abs(_decode(r, dtype)) > abs(value) else r


def _fill_ties_away(value, dtype):
    r = _orig_fill(value, dtype)
    lo = _orig_fill(math.nextafter(value, 0.0), dtype)
    hi = _orig_fill(math.nextafter(value, math.copysign(math.inf, value)), dtype)
    # at an exact tie the two neighbours disagree: take the one away from zero
    return hi if lo != hi and r == lo else r


def _loops_short(logits, bitmask, vocab_size, rows_to_apply, fill):
    _orig_loops(logits, bitmask, max(vocab_size - 1, 0), rows_to_apply, fill)


def _loops_tail_word_skipped(logits, bitmask, vocab_size, rows_to_apply, fill):
    _orig_loops(logits, bitmask, vocab_size - vocab_size % 32, rows_to_apply, fill)


MUTANTS = {
    "bit order msb first": ("get_bitmask_value", _bit_msb_first),
    "keep/mask sense inverted": ("get_bitmask_value", _bit_inverted),
    "word index j//16": ("get_bitmask_value", _bit_word_index_16),
    "mask row 0 for every row": ("get_bitmask_value", _bit_row_zero),
    "default vocab uses max": ("resolve_vocab_size", _vocab_max),
    "default vocab ignores mask width": ("resolve_vocab_size", _vocab_cols_only),
    "default vocab off by one": ("resolve_vocab_size", _vocab_off_by_one),
    "indices ignored": ("row_set", _rows_ignore_indices),
    "index position used as row": ("row_set", _rows_sorted_positions),
    "fill rounds toward zero": ("fill_bits", _fill_truncate),
    "fill ties away from zero": ("fill_bits", _fill_ties_away),
    "loop stops one short": ("apply_inplace_loops", _loops_short),
    "partial last word skipped": ("apply_inplace_loops", _loops_tail_word_skipped),
}


@pytest.mark.parametrize("name", list(MUTANTS))
def test_pins_reject_mutant(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(oracle, attr, fn)
    assert not pins_pass(), name
