"""Seeded synthetic inputs for the packed-bitmask apply.

This module only *draws* inputs: logits as raw bit patterns, packed int32
allow-masks, vocab sizes, row-index lists and fill values.  It holds none of
the apply arithmetic (no bit test, no masking, no fill conversion), so both
the HIP path and the CPU oracle can take their inputs from here without
sharing any of the method.

Five named workloads mirror the shapes the pages talk about:

* ``tiny``      -- fp32 [1, 32000], half the bits set, explicit vocab 32000.
* ``tail_bf16`` -- bf16 [8, 50257]: a vocab that is not a multiple of 32
                   (logits-processor page, "Correctness"), sparse allowed bits,
                   garbage in the padding bits of the last word (Modular MAX
                   ``apply_packed_bitmask``: padding bits are never read).
* ``mixed_bf16``-- bf16 [256, 128256] with an explicit vocab of 128000 and 128
                   random unique row indices (XGrammar "Bitmask Operations",
                   Notes: Padding and Indices); batch 256 x 128k vocab is the
                   shape the logits-processor page benchmarks.
* ``verify_fp16`` -- out-of-place fp16 [1024, 32000] with fill -65504: 256
                   slots x 4 speculative-verify rows (TensorRT-Edge-LLM
                   "Guided Decoder", ``applyMask`` over
                   [activeBatchSize, rowsPerSlot, vocab]), with 5 % all-zero
                   ("unsatisfiable") rows and 20 % all-ones rows.
* ``large_fp32`` -- fp32 [2048, 262144] with vocab 262100 and four row kinds.

Every workload takes size overrides so tests can draw the same structure at a
size a slow CPU oracle finishes quickly.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

# dtype name -> storage type of its bit patterns
BITS_DTYPE = {"float32": np.uint32, "float16": np.uint16, "bfloat16": np.uint16}
ELEM_BYTES = {"float32": 4, "float16": 2, "bfloat16": 2}


@dataclasses.dataclass
class Workload:
    """One apply problem, all arrays on the host as raw bit patterns."""

    name: str
    op: str                       # "inplace" or "out"
    dtype: str                    # "float32" | "float16" | "bfloat16"
    logits: np.ndarray            # uint32/uint16 [rows, cols] (bit patterns)
    mask: np.ndarray              # int32 [mask_rows, mask_cols]
    vocab_size: Optional[int]     # None -> the default rule
    indices: Optional[np.ndarray]  # int32 [n] or None
    fill_value: float
    out_init: Optional[np.ndarray] = None   # out-of-place: sentinel-filled output
    note: str = ""

    @property
    def rows(self) -> int:
        return self.logits.shape[0]

    @property
    def cols(self) -> int:
        return self.logits.shape[1]


# ----------------------------------------------------------------------------
# low-level draws
# ----------------------------------------------------------------------------

def normal_bits(rng: np.random.Generator, shape, sigma: float, dtype: str) -> np.ndarray:
    """N(0, sigma) logits drawn in fp32, stored as ``dtype`` bit patterns.

    bf16 is taken from the fp32 draw by round-to-nearest-even on the bit
    pattern (the draws are finite, so no NaN handling is needed).
    """
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    if dtype == "float32":
        return x.view(np.uint32)
    if dtype == "float16":
        return x.astype(np.float16).view(np.uint16)
    if dtype == "bfloat16":
        b = x.view(np.uint32)
        r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
        return r.astype(np.uint16)
    raise ValueError(dtype)


def pack_allowed(allowed: np.ndarray, mask_cols: int, rng: Optional[np.random.Generator],
                 garbage: bool = True) -> np.ndarray:
    """Pack a bool [rows, V] allow-array into int32 words, 32 tokens a word.

    Token v sits in word v // 32 at bit v % 32 (numpy's little-endian bit
    order on a little-endian host).  Bits past V in the last used word and all
    words past it up to ``mask_cols`` are filled with random garbage when
    ``garbage`` is set, else left zero.
    """
    rows, V = allowed.shape
    W = (V + 31) // 32
    assert mask_cols >= W
    padded = np.zeros((rows, W * 32), dtype=bool)
    padded[:, :V] = allowed
    words = np.packbits(padded, axis=1, bitorder="little").view("<u4").reshape(rows, W)
    out = np.zeros((rows, mask_cols), dtype=np.uint32)
    out[:, :W] = words
    if garbage and rng is not None:
        t = V % 32
        if t:
            junk = rng.integers(0, 2**32, size=rows, dtype=np.uint64).astype(np.uint32)
            keep_low = np.uint32((1 << t) - 1)
            out[:, W - 1] = (out[:, W - 1] & keep_low) | (junk & ~keep_low)
        if mask_cols > W:
            out[:, W:] = rng.integers(0, 2**32, size=(rows, mask_cols - W),
                                      dtype=np.uint64).astype(np.uint32)
    return out.view(np.int32)


def bernoulli_rows(rng: np.random.Generator, rows: int, V: int, density) -> np.ndarray:
    """bool [rows, V]; row i's bits are i.i.d. Bernoulli(density[i])."""
    d = np.broadcast_to(np.asarray(density, dtype=np.float64), (rows,))
    out = np.empty((rows, V), dtype=bool)
    # row blocks keep the float64 temporary small at large V
    step = max(1, (1 << 24) // max(V, 1))
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        out[r0:r1] = rng.random((r1 - r0, V)) < d[r0:r1, None]
    return out


# ----------------------------------------------------------------------------
# the five named workloads
# ----------------------------------------------------------------------------

def tiny(rows: int = 1, vocab: int = 32000, seed: int = 0) -> Workload:
    rng = np.random.Generator(np.random.PCG64(seed))
    W = (vocab + 31) // 32
    logits = normal_bits(rng, (rows, vocab), 1.0, "float32")
    mask = rng.integers(0, 2**32, size=(rows, W), dtype=np.uint64).astype(np.uint32).view(np.int32)
    return Workload("tiny", "inplace", "float32", logits, mask, vocab, None, -math.inf,
                    note="fp32 [1,32000] N(0,1), uniform random mask words, vocab_size=32000")


def tail_bf16(rows: int = 8, vocab: int = 50257, seed: int = 1) -> Workload:
    rng = np.random.Generator(np.random.PCG64(seed))
    W = (vocab + 31) // 32
    logits = normal_bits(rng, (rows, vocab), 3.0, "bfloat16")
    allowed = bernoulli_rows(rng, rows, vocab, 0.01)
    for r in range(rows):
        if not allowed[r].any():
            allowed[r, int(rng.integers(0, vocab))] = True
    mask = pack_allowed(allowed, W, rng, garbage=True)
    return Workload("tail_bf16", "inplace", "bfloat16", logits, mask, None, None, -math.inf,
                    note="bf16 [8,50257] N(0,3), density 0.01 (>=1 per row), garbage tail bits, "
                         "default vocab rule")


def mixed_bf16(rows: int = 256, vocab: int = 128000, col_pad: int = 256, word_pad: int = 8,
               n_indices: Optional[int] = None, seed: int = 2, sorted_indices: bool = False) -> Workload:
    rng = np.random.Generator(np.random.PCG64(seed))
    cols = vocab + col_pad
    W = (vocab + 31) // 32
    logits = normal_bits(rng, (rows, cols), 2.0, "bfloat16")
    dens = rng.uniform(0.001, 0.5, size=rows)
    allowed = bernoulli_rows(rng, rows, vocab, dens)
    mask = pack_allowed(allowed, W + word_pad, rng, garbage=True)
    n = rows // 2 if n_indices is None else n_indices
    idx = rng.permutation(rows)[:n].astype(np.int32)
    if sorted_indices:
        idx = np.sort(idx)
    return Workload("mixed_bf16", "inplace", "bfloat16", logits, mask, vocab, idx, -math.inf,
                    note=f"bf16 [{rows},{cols}] N(0,2), vocab_size={vocab} explicit, mask "
                         f"[{rows},{W + word_pad}], per-row density U[0.001,0.5], "
                         f"{n} unique random row indices")


def verify_fp16(slots: int = 256, rows_per_slot: int = 4, vocab: int = 32000, seed: int = 3) -> Workload:
    rng = np.random.Generator(np.random.PCG64(seed))
    rows = slots * rows_per_slot
    W = (vocab + 31) // 32
    logits = normal_bits(rng, (rows, vocab), 1.0, "float16")
    n_zero = int(round(0.05 * rows))
    n_ones = int(round(0.20 * rows))
    kind = np.full(rows, 2, dtype=np.int8)          # 2 = Bernoulli(0.05)
    perm = rng.permutation(rows)
    kind[perm[:n_zero]] = 0
    kind[perm[n_zero:n_zero + n_ones]] = 1
    allowed = bernoulli_rows(rng, rows, vocab, 0.05)
    allowed[kind == 0] = False
    allowed[kind == 1] = True
    mask = pack_allowed(allowed, W, rng, garbage=True)
    out_init = np.full((rows, vocab), 0x7E01, dtype=np.uint16)
    return Workload("verify_fp16", "out", "float16", logits, mask, None, None, -65504.0,
                    out_init=out_init,
                    note=f"out-of-place fp16 [{rows},{vocab}] ({slots} slots x {rows_per_slot} verify "
                         f"rows), fill -65504, density 0.05 with {n_zero} all-zero and "
                         f"{n_ones} all-ones rows")


def large_fp32(rows: int = 2048, cols: int = 262144, vocab: int = 262100, seed: int = 4,
               max_run: int = 4096) -> Workload:
    rng = np.random.Generator(np.random.PCG64(seed))
    mask_cols = (cols + 31) // 32
    W = (vocab + 31) // 32
    logits = normal_bits(rng, (rows, cols), 1.0, "float32")
    kind = np.arange(rows) % 4
    kind = kind[rng.permutation(rows)]
    mask = np.empty((rows, mask_cols), dtype=np.int32)
    step = max(1, (1 << 23) // vocab)
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        k = kind[r0:r1]
        n = r1 - r0
        allowed = np.zeros((n, vocab), dtype=bool)
        allowed[k == 0] = True
        sel = np.flatnonzero(k == 1)
        if sel.size:
            allowed[sel] = rng.random((sel.size, vocab)) < 0.3
        for i in np.flatnonzero(k == 2):
            L = int(rng.integers(1, min(max_run, vocab) + 1))
            s = int(rng.integers(0, vocab - L + 1))
            allowed[i, s:s + L] = True
        sel = np.flatnonzero(k == 3)
        if sel.size:
            allowed[sel] = rng.random((sel.size, vocab)) < 0.001
        mask[r0:r1] = pack_allowed(allowed, mask_cols, rng, garbage=True)
    assert W <= mask_cols
    return Workload("large_fp32", "inplace", "float32", logits, mask, vocab, None, -math.inf,
                    note=f"fp32 [{rows},{cols}] N(0,1), vocab_size={vocab}, four row kinds "
                         f"(all-ones, Bernoulli(0.3), one run of 1..{max_run}, Bernoulli(0.001))")


NAMED = {
    "tiny": tiny,
    "tail_bf16": tail_bf16,
    "mixed_bf16": mixed_bf16,
    "verify_fp16": verify_fp16,
    "large_fp32": large_fp32,
}


# ----------------------------------------------------------------------------
# fuzz cases
# ----------------------------------------------------------------------------

SPECIAL_BITS = {
    # a few patterns a kept logit must survive bit for bit
    "float32": [0x7FC00001, 0xFFC12345, 0x80000000, 0x00000001, 0x807FFFFF, 0x7F800000,
                0x7FBFFFFF],
    "float16": [0x7E01, 0xFC01, 0x8000, 0x0001, 0x83FF, 0x7C00, 0x7D55],
    "bfloat16": [0x7FC1, 0xFF81, 0x8000, 0x0001, 0x807F, 0x7F80, 0x7FA0],
}


def random_case(rng: np.random.Generator, dtype: str, rows: int, cols: int, *,
                row_pad: int = 0, mask_rows: Optional[int] = None,
                mask_cols: Optional[int] = None, mask_row_pad: int = 0,
                vocab_size: Optional[int] = None, n_indices: Optional[int] = None,
                density: float = 0.5, specials: bool = True, op: str = "inplace",
                fill_value: float = -math.inf):
    """A random problem with arbitrary padding; returns (Workload, stride, mask_stride).

    The logits are stored in a [rows, cols + row_pad] buffer (so the row pitch
    may break 16-byte alignment) and the mask in [mask_rows, mask_cols +
    mask_row_pad]; the Workload holds the *views* of width cols / mask_cols.
    """
    if mask_cols is None:
        mask_cols = (cols + 31) // 32
    if mask_rows is None:
        mask_rows = rows
    stride = cols + row_pad
    mstride = mask_cols + mask_row_pad
    buf = normal_bits(rng, (rows, stride), 1.0, dtype)
    if specials and rows * cols:
        sp = np.array(SPECIAL_BITS[dtype], dtype=BITS_DTYPE[dtype])
        k = max(1, rows * stride // 50)
        pos = rng.integers(0, rows * stride, size=k)
        buf.reshape(-1)[pos] = sp[rng.integers(0, sp.size, size=k)]
    mwords = rng.integers(0, 2**32, size=(mask_rows, mstride), dtype=np.uint64).astype(np.uint32)
    if density != 0.5:
        bits = rng.random((mask_rows, mstride * 32)) < density
        mwords = np.packbits(bits, axis=1, bitorder="little").view("<u4").reshape(mask_rows, mstride)
    mask_buf = mwords.view(np.int32)
    idx = None
    if n_indices is not None:
        limit = min(rows, mask_rows)
        idx = rng.permutation(limit)[:n_indices].astype(np.int32)
    wl = Workload("fuzz", op, dtype, buf[:, :cols], mask_buf[:, :mask_cols], vocab_size, idx,
                  fill_value)
    return wl, stride, mstride
