"""CPU oracle for the packed-bitmask apply.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product (the
HIP library and its Python binding) never imports, links or runs anything
here, and nothing here imports the product.

What the oracle computes, and where each piece comes from:

* ``get_bitmask_value`` -- row i's token j sits at bit ``j % 32`` of word
  ``j // 32``; a set bit keeps the token and a clear bit masks it.
  XGrammar "Bitmask Operations", apply_token_bitmask_inplace (a zero bit
  masks, a one bit keeps; the j-th bit of row i); Modular MAX
  "apply_packed_bitmask" (the bit-within-word and word-within-row rule).
  Words are int32 only for old-PyTorch reasons (XGrammar,
  allocate_token_bitmask), so they are read as uint32.
* ``resolve_vocab_size`` -- XGrammar "Bitmask Operations", Notes: Padding:
  a given vocab size restricts the op to logits[..., :V] and
  bitmask[..., :ceil(V/32)]; without one V = min(logits cols, 32 * mask cols).
* ``row_set`` -- XGrammar "Bitmask Operations", Notes: Indices: the listed
  rows only, batch sizes of logits and bitmask may then differ as long as the
  indices are valid; without indices every logits row.
* ``apply_inplace`` / ``apply_inplace_py`` -- the page's double loop: for each
  processed row, for each j < V, a zero bit writes the fill.  The C file
  ``apply_loop.c`` is that loop for large inputs; the pure-Python version is
  the same loop over lists for tiny inputs.
* ``apply_out`` -- Modular MAX "apply_packed_bitmask": output is the logit
  where the bit is set, else ``fill_value``.  Where an index list or a vocab
  size leaves part of the output outside the processed region, that part is
  a copy of the input (out-of-place = copy, then the in-place op).
* ``apply_rows`` -- TensorRT-Edge-LLM "Guided Decoder": the apply kernel
  leaves a row whose per-row flag is zero alone (``deviceRowNeedsMask``), and
  a row whose mask admits no token is unsatisfiable (``rowHasAnyToken``,
  ``fillMasks``' unsatisfiable slots).  Rows with a nonzero flag get the
  in-place op; the report is, per row, whether any of its first V tokens is
  still admitted afterwards: for a gated-off row that is simply V > 0 (the
  row is not masked), for the others whether any of bits [0, V) is set.
* ``fill_bits`` -- the fill as the dtype's bit pattern: the exact value of
  the double, rounded once to nearest-even in the target format (overflow to
  infinity, NaN to a quiet NaN with the input's sign and no payload).  The
  pages give the fill only as a value of the logits' dtype, so the rounding
  rule is a reading.

Everything works on raw bit patterns (uint16 for fp16/bf16, uint32 for
fp32); no logit is ever interpreted as a number.
"""

from __future__ import annotations

import ctypes
import math
import os
import pathlib
import subprocess
import tempfile
from fractions import Fraction
from typing import Optional, Sequence

import numpy as np

HERE = pathlib.Path(__file__).resolve().parent
C_SOURCE = HERE / "apply_loop.c"
C_LIBRARY = HERE / "_apply_loop.so"

# dtype -> (exponent bits, fraction bits) of the IEEE-style binary format
FORMATS = {"float32": (8, 23), "float16": (5, 10), "bfloat16": (8, 7)}
BITS_DTYPE = {"float32": np.uint32, "float16": np.uint16, "bfloat16": np.uint16}


# ----------------------------------------------------------------------------
# host-side rules
# ----------------------------------------------------------------------------

def resolve_vocab_size(cols: int, mask_cols: int, vocab_size: Optional[int] = None) -> int:
    """V for a [rows, cols] logits and a [mask_rows, mask_cols] bitmask.

    XGrammar "Bitmask Operations", Notes: Padding.  A given V must lie inside
    both tensors (it is the real vocab under possible padding of either).
    """
    limit = min(cols, 32 * mask_cols)
    if vocab_size is None:
        return limit
    if not (0 <= vocab_size <= limit):
        raise ValueError(f"vocab_size {vocab_size} outside [0, {limit}]")
    return int(vocab_size)


def row_set(rows: int, mask_rows: int, indices: Optional[Sequence[int]] = None) -> list:
    """Rows the op is applied to (XGrammar "Bitmask Operations", Notes: Indices)."""
    if indices is None:
        if mask_rows < rows:
            raise ValueError(f"bitmask has {mask_rows} rows for {rows} logits rows")
        return list(range(rows))
    out = []
    limit = min(rows, mask_rows)
    for i in indices:
        i = int(i)
        if not (0 <= i < limit):
            raise ValueError(f"index {i} outside [0, {limit})")
        out.append(i)
    return out


def fill_bits(value: float, dtype: str) -> int:
    """Bit pattern of ``value`` rounded once, to nearest-even, into ``dtype``.

    Works on the exact rational value of the double: find the binade, divide
    by the spacing of representable numbers there, round the quotient to an
    integer (ties to even), and encode.
    """
    ebits, mbits = FORMATS[dtype]
    width = 1 + ebits + mbits
    bias = (1 << (ebits - 1)) - 1
    exp_all = (1 << ebits) - 1
    sign_bit = (1 << (width - 1)) if math.copysign(1.0, value) < 0 else 0
    if math.isnan(value):
        return sign_bit | (exp_all << mbits) | (1 << (mbits - 1))
    if math.isinf(value):
        return sign_bit | (exp_all << mbits)
    a = Fraction(abs(value))
    if a == 0:
        return sign_bit
    # binade: 2**e <= a < 2**(e + 1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, 1 - bias)                 # below the normal range the spacing stays fixed
    n = a / Fraction(2) ** (e - mbits)   # value in units of the spacing
    m = n.numerator // n.denominator
    rest = n - m
    if rest > Fraction(1, 2) or (rest == Fraction(1, 2) and m % 2 == 1):
        m += 1
    if m < (1 << mbits):                 # subnormal result
        return sign_bit | m
    if m == (1 << (mbits + 1)):          # rounded up into the next binade
        m >>= 1
        e += 1
    exp_field = e + bias
    if exp_field >= exp_all:             # overflow
        return sign_bit | (exp_all << mbits)
    return sign_bit | (exp_field << mbits) | (m - (1 << mbits))


def get_bitmask_value(bitmask, i: int, j: int) -> int:
    """The j-th bit of row i: bit j % 32 of word j // 32, words read as uint32."""
    word = int(bitmask[i][j // 32]) & 0xFFFFFFFF
    return (word >> (j % 32)) & 1


# ----------------------------------------------------------------------------
# pure-Python literal loop (tiny inputs)
# ----------------------------------------------------------------------------

def apply_inplace_loops(logits: list, bitmask, vocab_size: int, rows_to_apply, fill: int) -> None:
    """XGrammar "Bitmask Operations", apply_token_bitmask_inplace, Notes: Indices.

    The double loop that page gives as the operation's definition, kept in
    its literal form over Python lists (``logits`` is a list of row lists):
    the oracle's rule for this op is to follow that loop as written.
    """
    for i in rows_to_apply:
        for j in range(vocab_size):
            if get_bitmask_value(bitmask, i, j) == 0:
                logits[i][j] = fill


def apply_inplace_py(logits: np.ndarray, mask: np.ndarray, dtype: str,
                     vocab_size: Optional[int] = None, indices=None,
                     fill_value: float = -math.inf) -> np.ndarray:
    """Pure-Python version of :func:`apply_inplace`; returns a new array."""
    rows, cols = logits.shape
    mask_rows, mask_cols = mask.shape
    V = resolve_vocab_size(cols, mask_cols, vocab_size)
    rs = row_set(rows, mask_rows, indices)
    fb = fill_bits(fill_value, dtype)
    rows_list = [[int(x) for x in row] for row in logits]
    mask_list = [[int(x) for x in row] for row in mask]
    apply_inplace_loops(rows_list, mask_list, V, rs, fb)
    return np.array(rows_list, dtype=logits.dtype).reshape(rows, cols)


# ----------------------------------------------------------------------------
# C literal loop (any size)
# ----------------------------------------------------------------------------

_lib = None


def build_c(target: pathlib.Path = C_LIBRARY) -> pathlib.Path:
    """Compile apply_loop.c with gcc (plain -O2, no vector flags)."""
    cmd = ["gcc", "-O2", "-std=c99", "-shared", "-fPIC", "-o", str(target), str(C_SOURCE)]
    subprocess.run(cmd, check=True)
    return target


def _load():
    global _lib
    if _lib is not None:
        return _lib
    so = C_LIBRARY
    if not so.exists() or so.stat().st_mtime < C_SOURCE.stat().st_mtime:
        try:
            build_c(so)
        except (OSError, subprocess.CalledProcessError):
            so = pathlib.Path(tempfile.mkdtemp(prefix="oracle_")) / "_apply_loop.so"
            build_c(so)
    lib = ctypes.CDLL(str(so))
    lib.oracle_rows_any_allowed.restype = None
    lib.oracle_rows_any_allowed.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                            ctypes.c_void_p]
    for name, ctype in (("oracle_apply_u32", ctypes.c_uint32), ("oracle_apply_u16", ctypes.c_uint16)):
        fn = getattr(lib, name)
        fn.restype = None
        fn.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                       ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctype]
    _lib = lib
    return lib


def _row_stride(a: np.ndarray) -> int:
    if a.ndim != 2 or a.strides[1] != a.itemsize:
        raise ValueError("need a 2-D array with a contiguous last dimension")
    if a.strides[0] % a.itemsize:
        raise ValueError("row stride is not a whole number of elements")
    return a.strides[0] // a.itemsize if a.shape[0] > 1 else max(a.shape[1], 1)


def apply_inplace(logits: np.ndarray, mask: np.ndarray, dtype: str,
                  vocab_size: Optional[int] = None, indices=None,
                  fill_value: float = -math.inf) -> np.ndarray:
    """In-place apply on a host array of bit patterns (returns ``logits``).

    ``logits`` is uint32 (fp32) or uint16 (fp16/bf16) [rows, cols], possibly
    a view of a wider buffer; ``mask`` is int32 [mask_rows, mask_cols],
    possibly a view too.
    """
    if logits.dtype != BITS_DTYPE[dtype]:
        raise TypeError(f"{dtype} logits must be stored as {BITS_DTYPE[dtype]}")
    if mask.dtype != np.int32:
        raise TypeError("bitmask must be int32")
    rows, cols = logits.shape
    mask_rows, mask_cols = mask.shape
    V = resolve_vocab_size(cols, mask_cols, vocab_size)
    rs = np.asarray(row_set(rows, mask_rows, indices), dtype=np.int64)
    fb = fill_bits(fill_value, dtype)
    if V == 0 or rs.size == 0:
        return logits
    lib = _load()
    fn = lib.oracle_apply_u32 if dtype == "float32" else lib.oracle_apply_u16
    fn(logits.ctypes.data, _row_stride(logits), mask.ctypes.data, _row_stride(mask),
       V, rs.ctypes.data, rs.size, fb)
    return logits


def apply_out(logits: np.ndarray, mask: np.ndarray, dtype: str,
              vocab_size: Optional[int] = None, indices=None,
              fill_value: float = -math.inf) -> np.ndarray:
    """Out-of-place apply: a fresh [rows, cols] array (copy, then in place)."""
    out = np.array(logits, copy=True, order="C")
    return apply_inplace(out, mask, dtype, vocab_size, indices, fill_value)


def rows_any_allowed(mask: np.ndarray, vocab_size: int) -> np.ndarray:
    """uint8 [mask_rows]: 1 where the row admits a token below ``vocab_size``."""
    if mask.dtype != np.int32:
        raise TypeError("bitmask must be int32")
    out = np.zeros(mask.shape[0], dtype=np.uint8)
    if mask.shape[0]:
        _load().oracle_rows_any_allowed(mask.ctypes.data, _row_stride(mask), int(vocab_size), mask.shape[0],
                                        out.ctypes.data)
    return out


def apply_rows(logits: np.ndarray, mask: np.ndarray, dtype: str, vocab_size: Optional[int] = None,
               row_needs_mask: Optional[np.ndarray] = None, fill_value: float = -math.inf):
    """Gated in-place apply plus the per-row report; returns (logits, any_allowed).

    ``row_needs_mask`` is one flag per logits row (None: every row); rows with
    a zero flag are left alone.  Needs mask_rows >= rows, as without indices.
    """
    rows, cols = logits.shape
    V = resolve_vocab_size(cols, mask.shape[1], vocab_size)
    if mask.shape[0] < rows:
        raise ValueError(f"bitmask has {mask.shape[0]} rows for {rows} logits rows")
    gate = np.ones(rows, dtype=np.int8) if row_needs_mask is None else np.asarray(row_needs_mask).reshape(rows)
    active = [r for r in range(rows) if gate[r] != 0]
    apply_inplace(logits, mask, dtype, V, active, fill_value)
    any_allowed = rows_any_allowed(mask[:rows], V)
    for r in range(rows):
        if gate[r] == 0:
            any_allowed[r] = 1 if V > 0 else 0
    return logits, any_allowed
