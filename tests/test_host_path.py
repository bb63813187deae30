"""The library's host-memory apply (CPU tensors) against the oracle, and the
XGrammar-compatible surface (XGrammar "Bitmask Operations").

The host path is native C++ in the same library (not the oracle, not
torch); these tests compare it bit for bit with the oracle on the same
seeded inputs, including strided views, index lists and the threaded path.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import packed_logit_bitmask_amd as mb
import workloads

TORCH = {"float32": (torch.int32, np.int32, torch.float32), "float16": (torch.int16, np.int16, torch.float16),
         "bfloat16": (torch.int16, np.int16, torch.bfloat16)}


def as_tensor(bits: np.ndarray, dtype: str):
    _, ndt, tdt = TORCH[dtype]
    return torch.from_numpy(bits.view(ndt)).view(tdt)


def bits_of(t, dtype: str) -> np.ndarray:
    idt, _, _ = TORCH[dtype]
    udt = np.uint32 if dtype == "float32" else np.uint16
    return t.view(idt).numpy().view(udt)


@pytest.mark.parametrize("name,kw", [
    ("tiny", {}), ("tail_bf16", {}), ("mixed_bf16", {}), ("verify_fp16", {}),
    ("large_fp32", {"rows": 16}),
])
def test_named_workloads(name, kw):
    wl = workloads.NAMED[name](**kw)
    if wl.op == "out":
        want = oracle.apply_out(wl.logits, wl.mask, wl.dtype, wl.vocab_size, wl.indices, wl.fill_value)
        got = mb.mi_apply_bitmask_out_host(as_tensor(wl.logits, wl.dtype), torch.from_numpy(wl.mask),
                                           vocab_size=wl.vocab_size, indices=wl.indices,
                                           fill_value=wl.fill_value)
    else:
        want = oracle.apply_inplace(wl.logits.copy(), wl.mask, wl.dtype, wl.vocab_size, wl.indices,
                                    wl.fill_value)
        x = wl.logits.copy()
        got = mb.mi_apply_bitmask_inplace_host(as_tensor(x, wl.dtype), torch.from_numpy(wl.mask),
                                               vocab_size=wl.vocab_size, indices=wl.indices,
                                               fill_value=wl.fill_value)
    assert np.array_equal(bits_of(got, wl.dtype), want)


@pytest.mark.parametrize("seed", range(24))
def test_fuzz_strided(seed):
    rng = np.random.default_rng(300 + seed)
    dtype = ["float32", "float16", "bfloat16"][seed % 3]
    rows = int(rng.integers(1, 12))
    cols = int(rng.integers(1, 900))
    mask_cols = (cols + 31) // 32 + int(rng.integers(0, 3))
    limit = min(cols, 32 * mask_cols)
    vocab = [None, int(rng.integers(0, limit + 1))][seed % 2]
    nidx = [None, 0, int(rng.integers(1, rows + 1))][seed % 3]
    wl, stride, mstride = workloads.random_case(rng, dtype, rows, cols, row_pad=int(rng.integers(0, 7)),
                                                mask_cols=mask_cols, mask_row_pad=int(rng.integers(0, 3)),
                                                vocab_size=vocab, n_indices=nidx,
                                                fill_value=float(rng.choice([-math.inf, -2.5])))
    want = oracle.apply_inplace(np.array(wl.logits), wl.mask, dtype, vocab, wl.indices, wl.fill_value)
    padded = np.zeros((rows, stride), dtype=wl.logits.dtype)   # a strided view, as in a padded tensor
    padded[:, :cols] = wl.logits
    view = padded[:, :cols]
    x = as_tensor(view, dtype)
    assert x.stride(0) == stride
    mb.mi_apply_bitmask_inplace_host(x, torch.from_numpy(wl.mask), vocab, wl.indices, wl.fill_value)
    assert np.array_equal(view, want)
    assert not padded[:, cols:].any()                          # padding columns untouched
    out = mb.mi_apply_bitmask_out_host(as_tensor(np.array(wl.logits), dtype), torch.from_numpy(wl.mask),
                                       vocab_size=vocab, indices=wl.indices, fill_value=wl.fill_value)
    assert np.array_equal(bits_of(out, dtype), want)


def test_threaded_rows_match():
    wl = workloads.mixed_bf16(rows=64, n_indices=48)      # > 2^20 elements: worker threads
    want = oracle.apply_inplace(wl.logits.copy(), wl.mask, wl.dtype, wl.vocab_size, wl.indices, wl.fill_value)
    for threads in (0, 1, 3, 64):
        x = as_tensor(wl.logits.copy(), wl.dtype)
        mb.mi_apply_bitmask_inplace_host(x, torch.from_numpy(wl.mask), wl.vocab_size, wl.indices,
                                         num_threads=threads)
        assert np.array_equal(bits_of(x, wl.dtype), want), threads


def test_threaded_rows_without_an_index_list():
    # every row, split over threads: each thread's rows start past row 0
    wl = workloads.mixed_bf16(rows=40, n_indices=8)
    want = oracle.apply_inplace(wl.logits.copy(), wl.mask, wl.dtype, wl.vocab_size, None, wl.fill_value)
    for threads in (2, 7, 40, 300):
        x = as_tensor(wl.logits.copy(), wl.dtype)
        mb.mi_apply_bitmask_inplace_host(x, torch.from_numpy(wl.mask), wl.vocab_size, None, num_threads=threads)
        assert np.array_equal(bits_of(x, wl.dtype), want), threads
        out = mb.mi_apply_bitmask_out_host(as_tensor(wl.logits.copy(), wl.dtype), torch.from_numpy(wl.mask),
                                           vocab_size=wl.vocab_size, fill_value=wl.fill_value, num_threads=threads)
        assert np.array_equal(bits_of(out, wl.dtype), want), threads


def test_host_checks_index_values():
    x = torch.zeros(4, 64, dtype=torch.float32)
    m = torch.zeros(3, 2, dtype=torch.int32)
    with pytest.raises(mb.BitmaskError) as e:
        mb.mi_apply_bitmask_inplace_host(x, m, indices=[0, 3])
    assert e.value.status == "MI_ERR_BAD_INDICES"
    assert torch.count_nonzero(x) == 0        # nothing written before the check


def test_host_binding_rejects_mismatched_tensors():
    x = torch.zeros(2, 64, dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        mb.mi_apply_bitmask_inplace_host(x, torch.zeros(2, 2, dtype=torch.int64))
    with pytest.raises(ValueError):
        mb.mi_apply_bitmask_out_host(x, torch.zeros(2, 2, dtype=torch.int32), out=torch.zeros(2, 64))
    with pytest.raises(ValueError):
        mb.mi_apply_bitmask_out_host(x, torch.zeros(2, 2, dtype=torch.int32),
                                     out=torch.zeros(2, 32, dtype=torch.bfloat16))


def test_xgrammar_surface_shapes_and_reset():
    assert mb.bitmask_dtype == torch.int32
    assert mb.get_bitmask_shape(8, 50257) == (8, 1571)
    assert mb.get_bitmask_shape(3, 32) == (3, 1)
    b = mb.allocate_token_bitmask(4, 100)
    assert b.shape == (4, 4) and b.dtype == torch.int32 and b.device.type == "cpu"
    assert torch.all(b == -1)
    b.zero_()
    mb.reset_token_bitmask(b)
    assert torch.all(b == -1)


@pytest.mark.parametrize("dtype", ["float32", "float16", "bfloat16"])
def test_xgrammar_apply_on_cpu_tensors(dtype):
    rng = np.random.default_rng(9)
    wl, _, _ = workloads.random_case(rng, dtype, 5, 333, mask_cols=12, n_indices=3, specials=False)
    want = oracle.apply_inplace(np.array(wl.logits), wl.mask, dtype, 300, list(wl.indices))
    x = as_tensor(np.array(wl.logits), dtype)
    mb.apply_token_bitmask_inplace(x, torch.from_numpy(np.ascontiguousarray(wl.mask)), vocab_size=300,
                                   indices=list(wl.indices))
    assert np.array_equal(bits_of(x, dtype), want)
    # an all-allowed freshly allocated mask is the identity
    x2 = as_tensor(np.array(wl.logits), dtype)
    mb.apply_token_bitmask_inplace(x2, mb.allocate_token_bitmask(5, 333))
    assert np.array_equal(bits_of(x2, dtype), np.array(wl.logits))


def test_host_loop_choice_and_the_portable_loop():
    """The host entry points run the AVX-512 loop where the CPU has it; the
    portable loop (forced through the environment, in a fresh process since
    the choice is made once) passes the same tests."""
    import os
    import subprocess
    import sys

    isa = mb.host_isa()
    assert isa in ("avx512", "portable")
    if os.environ.get("MI_BITMASK_HOST_ISA") == "portable":
        assert isa == "portable"
        return
    env = dict(os.environ, MI_BITMASK_HOST_ISA="portable")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", __file__],
                         env=env, capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stdout[-2000:] + res.stderr[-2000:]
