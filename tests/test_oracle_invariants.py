"""Properties the apply must have at any size, checked on the oracle.

(i)   fill count in the processed region == zero bits in range
      (inputs are finite normals, so no input equals the fill);
(ii)  non-processed rows and columns >= V keep their bits;
(iii) an all-ones mask is the identity;  (iv) an all-zero mask fills the
      whole processed region;  (v) padding bits and padding words change
      nothing;  (vi) applying twice equals applying once;  (vii) out of place
      equals copy + in place and leaves the input alone;  (viii) indices
      listing every row equal no indices, and any order of the indices gives
      the same result;  (ix) applying to a split of the rows equals applying
      to all of them.
"""

import math

import numpy as np
import pytest

import oracle
import workloads

CASES = [
    ("tiny", {}),
    ("tail_bf16", {}),
    ("mixed_bf16", {"rows": 48}),
    ("mixed_bf16", {"rows": 24, "vocab": 3000, "col_pad": 7, "word_pad": 3}),
    ("verify_fp16", {"slots": 64}),
    ("large_fp32", {"rows": 8, "cols": 20000, "vocab": 19990}),
]
IDS = [f"{n}-{i}" for i, (n, _) in enumerate(CASES)]


def zero_bits_in_range(mask_row, V):
    """Zero bits among tokens [0, V), counted word by word with int.bit_count."""
    n = 0
    full, tail = divmod(V, 32)
    for w in mask_row[:full].tolist():
        n += 32 - (w & 0xFFFFFFFF).bit_count()
    if tail:
        w = int(mask_row[full]) & ((1 << tail) - 1)
        n += tail - w.bit_count()
    return n


def run(wl, logits=None, mask=None, indices="same"):
    logits = wl.logits if logits is None else logits
    mask = wl.mask if mask is None else mask
    idx = wl.indices if isinstance(indices, str) else indices
    return oracle.apply_inplace(np.array(logits), mask, wl.dtype, wl.vocab_size, idx, wl.fill_value)


def processed(wl):
    return list(range(wl.rows)) if wl.indices is None else [int(i) for i in wl.indices]


@pytest.mark.parametrize("name,kw", CASES, ids=IDS)
def test_count_and_untouched(name, kw):
    wl = workloads.NAMED[name](**kw)
    V = oracle.resolve_vocab_size(wl.cols, wl.mask.shape[1], wl.vocab_size)
    fb = oracle.fill_bits(wl.fill_value, wl.dtype)
    out = run(wl)
    rows = processed(wl)
    for r in rows:
        assert int(np.count_nonzero(out[r, :V] == fb)) == zero_bits_in_range(wl.mask[r], V)
        assert np.array_equal(out[r, V:], wl.logits[r, V:])                          # (ii)
    others = sorted(set(range(wl.rows)) - set(rows))
    assert np.array_equal(out[others], wl.logits[others])                           # (ii)


@pytest.mark.parametrize("name,kw", CASES, ids=IDS)
def test_all_ones_all_zero_padding(name, kw):
    wl = workloads.NAMED[name](**kw)
    V = oracle.resolve_vocab_size(wl.cols, wl.mask.shape[1], wl.vocab_size)
    fb = oracle.fill_bits(wl.fill_value, wl.dtype)
    ones = np.full_like(wl.mask, -1)
    assert np.array_equal(run(wl, mask=ones), wl.logits)                            # (iii)
    zeros = np.zeros_like(wl.mask)
    out = run(wl, mask=zeros)
    for r in processed(wl):
        assert np.all(out[r, :V] == fb)                                              # (iv)
    # (v): flip every padding bit of the last used word and every padding word
    W, t = (V + 31) // 32, V % 32
    flipped = wl.mask.copy().view(np.uint32)
    if t:
        flipped[:, W - 1] ^= np.uint32((0xFFFFFFFF << t) & 0xFFFFFFFF)
    flipped[:, W:] ^= np.uint32(0xFFFFFFFF)
    assert np.array_equal(run(wl, mask=flipped.view(np.int32)), run(wl))


@pytest.mark.parametrize("name,kw", CASES, ids=IDS)
def test_idempotent_and_out_of_place(name, kw):
    wl = workloads.NAMED[name](**kw)
    once = run(wl)
    assert np.array_equal(run(wl, logits=once), once)                                # (vi)
    before = wl.logits.copy()
    out = oracle.apply_out(wl.logits, wl.mask, wl.dtype, wl.vocab_size, wl.indices, wl.fill_value)
    assert np.array_equal(out, once)                                                 # (vii)
    assert np.array_equal(wl.logits, before)


@pytest.mark.parametrize("name,kw", CASES, ids=IDS)
def test_index_forms_and_splits(name, kw):
    wl = workloads.NAMED[name](**kw)
    rng = np.random.default_rng(5)
    ref = run(wl)
    rows = processed(wl)
    if wl.indices is None:
        assert np.array_equal(run(wl, indices=list(range(wl.rows))), ref)            # (viii)
    perm = [rows[i] for i in rng.permutation(len(rows))]
    assert np.array_equal(run(wl, indices=perm), ref)                                # (viii)
    cut = len(rows) // 3
    part = run(wl, indices=rows[:cut])
    part = oracle.apply_inplace(part, wl.mask, wl.dtype, wl.vocab_size, rows[cut:], wl.fill_value)
    assert np.array_equal(part, ref)                                                 # (ix)
