"""Oracle against an independently written bit-string brute force.

The brute force spells each mask row out as a string of '0'/'1' characters,
token 0 first (bit 0 of word 0), and masks every token whose character is
'0' -- a different route to the same definition (XGrammar "Bitmask
Operations", apply_token_bitmask_inplace; Modular MAX "apply_packed_bitmask").
Exhaustive over every in-range bit pattern for one row of up to 9 tokens,
every vocab size, and every ordered index subset of up to 3 rows.
"""

import itertools

import numpy as np
import pytest

import oracle

DTYPES = ["float32", "float16", "bfloat16"]
BITS = {"float32": np.uint32, "float16": np.uint16, "bfloat16": np.uint16}


def brute(logits, mask, vocab, rows, fill):
    out = logits.copy()
    for i in rows:
        s = "".join(format(int(w) & 0xFFFFFFFF, "032b")[::-1] for w in mask[i])
        for j in range(vocab):
            if s[j] == "0":
                out[i, j] = fill
    return out


def rand_logits(rng, dtype, rows, cols):
    hi = 2**32 if BITS[dtype] == np.uint32 else 2**16
    return rng.integers(0, hi, size=(rows, cols), dtype=np.uint64).astype(BITS[dtype])


@pytest.mark.parametrize("cols", range(1, 10))
def test_exhaustive_single_row(cols):
    rng = np.random.default_rng(cols)
    dtype = DTYPES[cols % 3]
    fill = oracle.fill_bits(-np.inf, dtype)
    logits = rand_logits(rng, dtype, 1, cols)
    for pattern in range(1 << cols):
        garbage = int(rng.integers(0, 2**32)) & ~((1 << cols) - 1) & 0xFFFFFFFF
        mask = np.array([[pattern | garbage]], dtype=np.uint64).astype(np.uint32).view(np.int32)
        for vocab in list(range(cols + 1)) + [None]:
            V = cols if vocab is None else vocab
            want = brute(logits, mask, V, [0], fill)
            got_c = oracle.apply_inplace(logits.copy(), mask, dtype, vocab_size=vocab)
            assert np.array_equal(got_c, want), (pattern, vocab)
            if pattern % 7 == 0:
                got_py = oracle.apply_inplace_py(logits, mask, dtype, vocab_size=vocab)
                assert np.array_equal(got_py, want), (pattern, vocab)


@pytest.mark.parametrize("dtype", DTYPES)
def test_every_ordered_index_subset(dtype):
    rng = np.random.default_rng(7)
    rows, cols, mask_cols = 3, 45, 2
    logits = rand_logits(rng, dtype, rows, cols)
    mask = rng.integers(0, 2**32, size=(rows, mask_cols), dtype=np.uint64).astype(np.uint32).view(np.int32)
    fill = oracle.fill_bits(-7.25, dtype)
    for k in range(rows + 1):
        for subset in itertools.permutations(range(rows), k):
            want = brute(logits, mask, cols, list(subset), fill)
            got = oracle.apply_inplace(logits.copy(), mask, dtype, indices=list(subset), fill_value=-7.25)
            assert np.array_equal(got, want), subset
            got_py = oracle.apply_inplace_py(logits, mask, dtype, indices=list(subset), fill_value=-7.25)
            assert np.array_equal(got_py, want), subset


@pytest.mark.parametrize("seed", range(6))
def test_random_multiword_rows(seed):
    rng = np.random.default_rng(100 + seed)
    dtype = DTYPES[seed % 3]
    rows = int(rng.integers(1, 5))
    cols = int(rng.integers(1, 200))
    mask_cols = (cols + 31) // 32 + int(rng.integers(0, 3))
    mask_rows = rows + int(rng.integers(0, 3))
    vocab = int(rng.integers(0, min(cols, 32 * mask_cols) + 1))
    logits = rand_logits(rng, dtype, rows, cols)
    mask = rng.integers(0, 2**32, size=(mask_rows, mask_cols), dtype=np.uint64).astype(np.uint32).view(np.int32)
    fill = oracle.fill_bits(-np.inf, dtype)
    want = brute(logits, mask, vocab, range(rows), fill)
    assert np.array_equal(oracle.apply_inplace(logits.copy(), mask, dtype, vocab_size=vocab), want)
    assert np.array_equal(oracle.apply_inplace_py(logits, mask, dtype, vocab_size=vocab), want)
    # out of place: a fresh array with the same content, input untouched
    before = logits.copy()
    assert np.array_equal(oracle.apply_out(logits, mask, dtype, vocab_size=vocab), want)
    assert np.array_equal(logits, before)
