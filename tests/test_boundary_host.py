"""The C ABI on a host without a GPU: exports, host helpers, argument checks.

Every call here either runs a pure host helper or is rejected by the
library's argument checks, which run before any HIP call, so nothing touches
a device.  Dummy pointers are never dereferenced on these paths.
"""

import ctypes
import math
import pathlib
import re

import numpy as np
import pytest

import oracle
import packed_logit_bitmask_amd as mb
from packed_logit_bitmask_amd import _binding

HEADER = pathlib.Path(__file__).resolve().parents[1] / "include" / "mi_bitmask.h"

OK, NULLP, DTYPE, SHAPE, VOCAB, INDICES, ALIAS, HIP, MISALIGNED, VARIANT = range(10)

LOGITS = 0x7F0000000000
MASK = 0x7F1000000000
IDX = 0x7F2000000000
OUT = 0x7F3000000000


def declared_functions():
    text = HEADER.read_text()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(mi_\w+)\s*\(", text, re.M)))


def test_exports_match_header():
    lib = mb.load_library()
    names = declared_functions()
    assert names == sorted(_binding.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(ImportError):
        _binding.load_library(tmp_path / "nope.so")


def test_status_strings():
    lib = mb.load_library()
    for code, name in enumerate(_binding.STATUS):
        assert lib.mi_status_string(code).decode() == name
    assert lib.mi_status_string(99).decode() == "MI_ERR_UNKNOWN"


def test_status_values_match_header():
    """The binding's status names sit at the values the header gives them,
    and the first eight are the boundary's list in its order (MI_ERR_HIP = 7),
    with the two codes added later after it."""
    text = HEADER.read_text()
    body = text[text.index("typedef enum mi_status"):]
    body = body[:body.index("} mi_status_t;")]
    values = {m.group(1): int(m.group(2)) for m in re.finditer(r"(MI_\w+)\s*=\s*(\d+)", body)}
    assert values == {name: code for code, name in enumerate(_binding.STATUS)}
    assert _binding.STATUS[:8] == ["MI_OK", "MI_ERR_NULL_POINTER", "MI_ERR_BAD_DTYPE", "MI_ERR_BAD_SHAPE",
                                   "MI_ERR_BAD_VOCAB", "MI_ERR_BAD_INDICES", "MI_ERR_ALIAS", "MI_ERR_HIP"]


@pytest.mark.parametrize("dtype", ["float32", "float16", "bfloat16"])
def test_fill_bits_match_oracle(dtype):
    rng = np.random.default_rng(21)
    vals = np.concatenate([
        rng.standard_normal(3000) * 10.0 ** rng.integers(-45, 40, size=3000),
        rng.standard_normal(1000) * 2.0 ** -24, rng.standard_normal(1000) * 2.0 ** -135,
        rng.uniform(-7e4, 7e4, 1000), [0.0, -0.0, math.inf, -math.inf, 65504.0, -65504.0, 65520.0,
                                       3.4028235677973366e38, 1e-320, 2.0 ** -149, 2.0 ** -150,
                                       1 + 2.0 ** -8, 1 + 2.0 ** -8 + 2.0 ** -30],
    ])
    for v in vals.tolist():
        assert mb.fill_value_bits(v, dtype) == oracle.fill_bits(v, dtype), (v, dtype)
    assert mb.fill_value_bits(math.nan, dtype) == oracle.fill_bits(math.nan, dtype)
    assert mb.fill_value_bits(-math.nan, dtype) == oracle.fill_bits(-math.nan, dtype)


def test_fill_bits_every_half_pattern_round_trips():
    pats = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = pats.view(np.float16).astype(np.float64)
    for p, v in zip(pats.tolist(), vals.tolist()):
        if math.isfinite(v):
            assert mb.fill_value_bits(v, "float16") == p


def test_resolve_vocab_matches_oracle():
    rng = np.random.default_rng(22)
    for _ in range(3000):
        cols = int(rng.integers(0, 300))
        mcols = int(rng.integers(0, 12))
        v = int(rng.integers(-3, 330)) if rng.random() < 0.8 else None
        try:
            want = oracle.resolve_vocab_size(cols, mcols, v if (v is None or v != -1) else None)
            if v is not None and v < -1:
                want = "err"
        except ValueError:
            want = "err"
        try:
            got = mb.resolve_vocab_size(cols, mcols, v)
        except mb.BitmaskError as e:
            assert e.status == "MI_ERR_BAD_VOCAB"
            got = "err"
        assert got == want, (cols, mcols, v)


def inplace(**kw):
    a = dict(logits=LOGITS, dtype=2, rows=4, cols=100, ls=100, mask=MASK, mask_rows=4, mask_cols=4, ms=4,
             vocab=-1, indices=None, n=0, fill=-math.inf, variant=None)
    a.update(kw)
    lib = mb.load_library()
    args = (a["logits"], a["dtype"], a["rows"], a["cols"], a["ls"], a["mask"], a["mask_rows"],
            a["mask_cols"], a["ms"], a["vocab"], a["indices"], a["n"], a["fill"])
    if a["variant"] is None:
        return lib.mi_apply_bitmask_inplace(*args, None)
    return lib.mi_apply_bitmask_inplace_ex(*args, a["variant"], None)


def outofplace(**kw):
    a = dict(out=OUT, os=100, logits=LOGITS, dtype=1, rows=4, cols=100, ls=100, mask=MASK, mask_rows=4,
             mask_cols=4, ms=4, vocab=-1, indices=None, n=0, fill=-1.0, variant=None)
    a.update(kw)
    lib = mb.load_library()
    args = (a["out"], a["os"], a["logits"], a["dtype"], a["rows"], a["cols"], a["ls"], a["mask"],
            a["mask_rows"], a["mask_cols"], a["ms"], a["vocab"], a["indices"], a["n"], a["fill"])
    if a["variant"] is None:
        return lib.mi_apply_bitmask_out(*args, None)
    return lib.mi_apply_bitmask_out_ex(*args, a["variant"], None)


REJECT_INPLACE = [
    ("null logits", dict(logits=None), NULLP),
    ("null mask", dict(mask=None), NULLP),
    ("null logits with rows but empty mask", dict(logits=None, mask=None, mask_cols=0), NULLP),
    ("indices NULL with count", dict(indices=None, n=3), NULLP),
    ("bad dtype", dict(dtype=3), DTYPE),
    ("negative dtype", dict(dtype=-1), DTYPE),
    ("negative rows", dict(rows=-1), SHAPE),
    ("negative cols", dict(cols=-5), SHAPE),
    ("negative mask rows", dict(mask_rows=-1), SHAPE),
    ("stride below cols", dict(ls=99), SHAPE),
    ("mask stride below width", dict(ms=3), SHAPE),
    ("too few mask rows", dict(mask_rows=3), SHAPE),
    ("cols above 2^30", dict(cols=(1 << 30) + 1, ls=(1 << 30) + 1), SHAPE),
    ("vocab above cols", dict(vocab=101), VOCAB),
    ("vocab above mask bits", dict(cols=200, ls=200, vocab=129), VOCAB),
    ("vocab below -1", dict(vocab=-2), VOCAB),
    ("negative index count", dict(indices=IDX, n=-1), INDICES),
    ("misaligned bf16 logits", dict(logits=LOGITS + 1), MISALIGNED),
    ("misaligned fp32 logits", dict(dtype=0, logits=LOGITS + 2), MISALIGNED),
    ("misaligned mask", dict(mask=MASK + 2), MISALIGNED),
    ("misaligned indices", dict(indices=IDX + 2, n=2), MISALIGNED),
    ("mask inside logits", dict(mask=LOGITS + 64), ALIAS),
    ("logits end overlaps mask start", dict(mask=LOGITS + 796), ALIAS),
    ("indices inside logits", dict(indices=LOGITS + 16, n=2), ALIAS),
    ("unknown variant", dict(variant=7), VARIANT),
    ("extent overflow", dict(rows=1 << 30, ls=1 << 40, cols=100, mask_rows=1 << 30), SHAPE),
]


@pytest.mark.parametrize("name,kw,code", REJECT_INPLACE, ids=[r[0] for r in REJECT_INPLACE])
def test_inplace_rejections(name, kw, code):
    assert inplace(**kw) == code
    assert mb.load_library().mi_last_error_message().decode()


def test_null_is_fine_for_empty_buffers():
    # checked through a later error so that nothing is launched
    assert inplace(logits=None, rows=0, mask=None, mask_rows=0, variant=7) == VARIANT
    assert inplace(logits=None, cols=0, ls=0, variant=7) == VARIANT
    assert outofplace(out=None, logits=None, rows=0, mask_rows=0, variant=3) == VARIANT


def test_adjacent_buffers_are_not_aliases():
    # logits [4,100] bf16 span [LOGITS, LOGITS + 800).  Buffers that touch
    # but do not overlap pass the alias checks; the unknown variant, checked
    # after them, then stops the call before any launch.
    assert inplace(mask=LOGITS + 800, variant=7) == VARIANT
    assert inplace(mask=LOGITS - 64, variant=7) == VARIANT     # mask is 4 x 4 words = 64 bytes
    assert inplace(mask=LOGITS - 60, variant=7) == ALIAS
    assert inplace(indices=LOGITS + 800, n=4, variant=7) == VARIANT
    assert outofplace(out=LOGITS + 800, os=100, dtype=2, variant=3) == VARIANT


REJECT_OUT = [
    ("null out", dict(out=None), NULLP),
    ("wronly has no out form", dict(variant=3), VARIANT),
    ("resident variant has no out form", dict(variant=4), VARIANT),
    ("out stride below cols", dict(os=50), SHAPE),
    ("misaligned out", dict(out=OUT + 1), MISALIGNED),
    ("out overlaps logits", dict(out=LOGITS + 10), ALIAS),
    ("out overlaps mask", dict(out=MASK - 100), ALIAS),
    ("out overlaps indices", dict(indices=OUT + 64, n=4), ALIAS),
    ("in-place through out checks mask alias", dict(out=LOGITS, mask=LOGITS + 8), ALIAS),
    ("bad dtype", dict(dtype=9), DTYPE),
    ("vocab above mask bits", dict(vocab=129), VOCAB),
]


@pytest.mark.parametrize("name,kw,code", REJECT_OUT, ids=[r[0] for r in REJECT_OUT])
def test_out_rejections(name, kw, code):
    assert outofplace(**kw) == code
    assert mb.load_library().mi_last_error_message().decode()


def test_binding_rejects_cpu_tensors_and_bad_indices():
    import torch
    x = torch.zeros(2, 64, dtype=torch.bfloat16)
    m = torch.zeros(2, 2, dtype=torch.int32)
    with pytest.raises(ValueError):
        mb.mi_apply_bitmask_inplace(x, m)
    with pytest.raises(ValueError):
        mb.mi_apply_bitmask_out(x, m)


def rows_call(**kw):
    a = dict(logits=LOGITS, dtype=2, rows=4, cols=100, ls=100, mask=MASK, mask_rows=4, mask_cols=4, ms=4,
             vocab=-1, gate=None, out=None, fill=-math.inf)
    a.update(kw)
    return mb.load_library().mi_apply_bitmask_rows(
        a["logits"], a["dtype"], a["rows"], a["cols"], a["ls"], a["mask"], a["mask_rows"], a["mask_cols"],
        a["ms"], a["vocab"], a["gate"], a["out"], a["fill"], None)


REJECT_ROWS = [
    ("null logits", dict(logits=None), NULLP),
    ("too few mask rows", dict(mask_rows=3), SHAPE),
    ("vocab too large", dict(vocab=129), VOCAB),
    ("gate inside logits", dict(gate=LOGITS + 10), ALIAS),
    ("report inside logits", dict(out=LOGITS + 100), ALIAS),
    ("report inside mask", dict(out=MASK + 8), ALIAS),
    ("report overlaps gate", dict(gate=OUT, out=OUT + 2), ALIAS),
    ("mask inside logits", dict(mask=LOGITS + 64), ALIAS),
]


@pytest.mark.parametrize("name,kw,code", REJECT_ROWS, ids=[r[0] for r in REJECT_ROWS])
def test_rows_rejections(name, kw, code):
    assert rows_call(**kw) == code
    assert mb.load_library().mi_last_error_message().decode()


def sample_call(**kw):
    a = dict(logits=LOGITS, dtype=2, rows=4, cols=100, ls=100, mask=MASK, mask_rows=4, mask_cols=4, ms=4,
             vocab=-1, tokens=OUT, params=True)
    a.update(kw)
    prm = _binding.SampleParams()
    prm.temperature_all, prm.top_k_all, prm.top_p_all, prm.min_p_all = 1.0, 0, 1.0, 0.0
    for name in ("temperature", "top_k", "top_p", "min_p"):
        if name in kw:
            setattr(prm, name, kw[name])
    return mb.load_library().mi_apply_bitmask_sample(
        a["logits"], a["dtype"], a["rows"], a["cols"], a["ls"], a["mask"], a["mask_rows"], a["mask_cols"],
        a["ms"], a["vocab"], ctypes.byref(prm) if a["params"] else None, a["tokens"], None)


REJECT_SAMPLE = [
    ("null params", dict(params=False), NULLP),
    ("null tokens", dict(tokens=None), NULLP),
    ("null logits", dict(logits=None), NULLP),
    ("bad dtype", dict(dtype=7), DTYPE),
    ("too few mask rows", dict(mask_rows=3), SHAPE),
    ("vocab too large for the mask", dict(vocab=129), VOCAB),
    ("vocab above 2^28 without a mask", dict(mask=None, rows=1, cols=(1 << 28) + 8, ls=(1 << 28) + 8,
                                             vocab=(1 << 28) + 1), SHAPE),
    ("tokens inside logits", dict(tokens=LOGITS + 16), ALIAS),
    ("tokens inside mask", dict(tokens=MASK + 8), ALIAS),
    ("tokens misaligned", dict(tokens=OUT + 4), MISALIGNED),
    ("per-row temperature misaligned", dict(temperature=IDX + 2), MISALIGNED),
]


@pytest.mark.parametrize("name,kw,code", REJECT_SAMPLE, ids=[r[0] for r in REJECT_SAMPLE])
def test_sample_rejections(name, kw, code):
    assert sample_call(**kw) == code
    assert mb.load_library().mi_last_error_message().decode()


def test_sample_accepts_the_largest_vocab_at_the_checks():
    """2^28 passes the size checks; with zero rows nothing is launched."""
    assert sample_call(mask=None, rows=0, cols=1 << 28, ls=1 << 28, vocab=1 << 28) == OK


def sample_ws_call(workspace, workspace_bytes, **kw):
    """A bf16 batch the workspace can split (4 rows of 8192 tokens, top-k 50)."""
    a = dict(logits=LOGITS, dtype=2, rows=4, cols=8192, ls=8192, mask=MASK, mask_rows=4, mask_cols=256, ms=256,
             vocab=-1, tokens=OUT)
    a.update(kw)
    prm = _binding.SampleParams()
    prm.temperature_all, prm.top_k_all, prm.top_p_all, prm.min_p_all = 1.0, 50, 1.0, 0.0
    for name in ("temperature", "top_k", "top_p", "min_p"):
        if name in kw:
            setattr(prm, name, kw[name])
    return mb.load_library().mi_apply_bitmask_sample_ws(
        a["logits"], a["dtype"], a["rows"], a["cols"], a["ls"], a["mask"], a["mask_rows"], a["mask_cols"],
        a["ms"], a["vocab"], ctypes.byref(prm), a["tokens"], workspace, workspace_bytes, None)


WS = 0x7F4000000000
WS_BYTES = 4 * 262288

REJECT_SAMPLE_WS = [
    ("negative workspace bytes", dict(workspace=WS, workspace_bytes=-1), SHAPE),
    ("workspace misaligned", dict(workspace=WS + 8, workspace_bytes=WS_BYTES), MISALIGNED),
    ("workspace over logits", dict(workspace=LOGITS + 4096, workspace_bytes=WS_BYTES), ALIAS),
    ("workspace over mask", dict(workspace=MASK - 16, workspace_bytes=WS_BYTES), ALIAS),
    ("workspace over tokens", dict(workspace=OUT - 1024, workspace_bytes=WS_BYTES), ALIAS),
    ("workspace over a per-row array", dict(workspace=WS, workspace_bytes=WS_BYTES, top_p=WS + 4096), ALIAS),
]


@pytest.mark.parametrize("name,kw,code", REJECT_SAMPLE_WS, ids=[r[0] for r in REJECT_SAMPLE_WS])
def test_sample_ws_rejections(name, kw, code):
    kw = dict(kw)
    assert sample_ws_call(kw.pop("workspace"), kw.pop("workspace_bytes"), **kw) == code
    assert mb.load_library().mi_last_error_message().decode()


def test_sample_ws_checks_only_a_workspace_it_uses():
    """A workspace that is too small, or a batch that cannot split (fp32, more
    than 32 rows, fewer than 8192 tokens), leaves the workspace unused: its
    placement is not checked, and with zero rows nothing is launched."""
    assert sample_ws_call(LOGITS + 4096, WS_BYTES - 1, rows=0) == OK
    assert sample_ws_call(LOGITS + 4096, WS_BYTES, dtype=0, rows=0) == OK
    assert sample_ws_call(WS + 8, WS_BYTES, rows=0, cols=8191, ls=8191) == OK
    assert sample_ws_call(WS + 8, WS_BYTES, rows=0) == OK            # no rows: nothing to split


def test_sample_workspace_bytes():
    lib = mb.load_library()
    per_row = 65536 * 4 + 128 + 16
    assert lib.mi_sample_workspace_bytes(2, 1, 128000) == per_row
    assert lib.mi_sample_workspace_bytes(1, 32, 8192) == 32 * per_row
    assert lib.mi_sample_workspace_bytes(1, 33, 8192) == 0       # more rows than the split takes
    # more rows than compute units, rows longer than a 512-thread block holds in
    # registers: one bit per row (rounded up to 256 bytes) orders them heavy first
    assert lib.mi_sample_workspace_bytes(1, 256, 32000) == 0
    assert lib.mi_sample_workspace_bytes(1, 257, 16385) == 256
    assert lib.mi_sample_workspace_bytes(1, 1024, 16384) == 0    # rows held in registers are not ordered
    assert lib.mi_sample_workspace_bytes(2, 1024, 32000) == 256
    assert lib.mi_sample_workspace_bytes(2, 8192, 65536) == 1024
    assert lib.mi_sample_workspace_bytes(2, 8193, 65536) == 0    # beyond the ordered rows
    assert lib.mi_sample_workspace_bytes(2, 1024, 65537) == 256  # rows of the 16-bit-counter search too
    assert lib.mi_sample_workspace_bytes(1, 300, 1 << 20) == 256
    assert lib.mi_sample_workspace_bytes(0, 1024, 32000) == 0    # fp32 rows
    assert lib.mi_sample_workspace_bytes(2, 16, 8191) == 0       # rows too short to split
    assert lib.mi_sample_workspace_bytes(0, 16, 128000) == 0     # fp32 rows are not split
    assert lib.mi_sample_workspace_bytes(7, 16, 128000) == 0     # invalid dtype
    assert lib.mi_sample_workspace_bytes(2, 0, 128000) == 0
    assert lib.mi_sample_workspace_bytes(2, 1, (1 << 28) + 1) == 0
    torch = pytest.importorskip("torch")
    assert mb.sample_workspace_bytes(torch.float16, 3, 32000) == 3 * per_row
