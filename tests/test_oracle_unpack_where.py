"""Oracle against the library route the fused op replaces.

Modular MAX "apply_packed_bitmask" describes the fused apply as replacing a
CPU unpack of the bitmask followed by a where().  numpy's
``unpackbits(..., bitorder="little")`` on the little-endian bytes of the
int32 words yields token 0 first, so ``where(keep, logits, fill)`` on that
unpacked mask must equal the oracle on every input.
"""

import math

import numpy as np
import pytest

import oracle
import workloads

DTYPES = ["float32", "float16", "bfloat16"]


def unpack_where(logits, mask, dtype, vocab, rows, fill_value):
    m = np.ascontiguousarray(mask)
    keep = np.unpackbits(m.view(np.uint8), axis=1, bitorder="little")[:, :vocab].astype(bool)
    fill = oracle.fill_bits(fill_value, dtype)
    out = np.array(logits, copy=True)
    rows = np.asarray(list(rows), dtype=np.int64)
    if rows.size and vocab:
        out[rows, :vocab] = np.where(keep[rows], logits[rows, :vocab], logits.dtype.type(fill))
    return out


def test_numpy_bit_order_matches_pages():
    # word 1 -> token 0 only; INT32_MIN -> token 31 only (LSB-first tokens in each word)
    m = np.array([[1, -(2**31)]], dtype=np.int32)
    u = np.unpackbits(m.view(np.uint8), axis=1, bitorder="little")
    assert u[0, 0] == 1 and u[0, 1:32].sum() == 0
    assert u[0, 63] == 1 and u[0, 32:63].sum() == 0


@pytest.mark.parametrize("seed", range(12))
def test_random_padded_views(seed):
    rng = np.random.default_rng(seed)
    dtype = DTYPES[seed % 3]
    rows = int(rng.integers(1, 9))
    cols = int(rng.integers(1, 700))
    mask_cols = (cols + 31) // 32 + int(rng.integers(0, 4))
    with_idx = seed % 2 == 1
    wl, _, _ = workloads.random_case(
        rng, dtype, rows, cols, row_pad=int(rng.integers(0, 9)),
        mask_rows=rows + int(rng.integers(0, 3)), mask_cols=mask_cols,
        mask_row_pad=int(rng.integers(0, 3)),
        n_indices=int(rng.integers(0, rows + 1)) if with_idx else None,
        density=float(rng.choice([0.5, 0.03, 0.97])))
    limit = min(cols, 32 * mask_cols)
    vocab = None if seed % 3 == 0 else int(rng.integers(0, limit + 1))
    V = oracle.resolve_vocab_size(cols, mask_cols, vocab)
    rowsel = range(rows) if wl.indices is None else wl.indices
    want = unpack_where(wl.logits, wl.mask, dtype, V, rowsel, -math.inf)
    got = oracle.apply_inplace(np.array(wl.logits), wl.mask, dtype, vocab, wl.indices)
    assert np.array_equal(got, want)
    got_out = oracle.apply_out(wl.logits, wl.mask, dtype, vocab, wl.indices, fill_value=-3.5)
    assert np.array_equal(got_out, unpack_where(wl.logits, wl.mask, dtype, V, rowsel, -3.5))


@pytest.mark.parametrize("name,kw", [
    ("tiny", {}),
    ("tail_bf16", {}),
    ("mixed_bf16", {"rows": 32}),
    ("verify_fp16", {"slots": 32}),
    ("large_fp32", {"rows": 8, "cols": 8192, "vocab": 8150}),
])
def test_named_workloads(name, kw):
    wl = workloads.NAMED[name](**kw)
    V = oracle.resolve_vocab_size(wl.cols, wl.mask.shape[1], wl.vocab_size)
    rowsel = range(wl.rows) if wl.indices is None else wl.indices
    want = unpack_where(wl.logits, wl.mask, wl.dtype, V, rowsel, wl.fill_value)
    if wl.op == "out":
        got = oracle.apply_out(wl.logits, wl.mask, wl.dtype, wl.vocab_size, wl.indices, wl.fill_value)
    else:
        got = oracle.apply_inplace(wl.logits.copy(), wl.mask, wl.dtype, wl.vocab_size, wl.indices,
                                   wl.fill_value)
    assert np.array_equal(got, want)
