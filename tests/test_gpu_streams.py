"""Calls on a side stream whose arguments need conversion by the binding.

The binding turns int64 index tensors, bool gates and float64 per-row
sampler parameters into the int32 / int8 / float32 device arrays the C ABI
takes, and allocates outputs (the per-row report, the sampled tokens).  With
``stream=s`` all of that must be enqueued on ``s`` ahead of the library's
kernels: here the current stream is kept busy by a bounded spin while the
call runs on ``s``, so a conversion left on the current stream would land
after the kernel that reads it.  Freed int32 / float32 blocks holding
invalid values are left in the allocator's cache first, so a kernel that
ran early would read those rather than the right values.
"""

import sys

import numpy as np
import pytest

import oracle
import workloads
import packed_logit_bitmask_amd as mb

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

SPIN_CYCLES = 20_000_000   # a bounded spin on the current stream


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu-marked tests need an MI355X")
    mb.load_library()


def poison_cache(n, dtype, value):
    """Leave a freed block of n elements of `dtype` holding `value` in the cache."""
    t = torch.full((n,), value, dtype=dtype, device="cuda")
    torch.cuda.synchronize()
    del t


def busy_current_stream():
    torch.cuda._sleep(SPIN_CYCLES)


def bf16_bits_to_device(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda").view(torch.bfloat16)


def test_inplace_int64_indices_on_side_stream():
    say("[gpu] side stream: int64 device indices")
    wl = workloads.mixed_bf16(rows=32, vocab=6000, col_pad=8, word_pad=1, n_indices=20)
    want = wl.logits.copy()
    oracle.apply_inplace(want, wl.mask, wl.dtype, wl.vocab_size, list(wl.indices), wl.fill_value)
    d = bf16_bits_to_device(wl.logits)
    dm = torch.from_numpy(wl.mask).to("cuda")
    idx64 = torch.from_numpy(wl.indices.astype(np.int64)).to("cuda")
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    poison_cache(idx64.numel(), torch.int32, -1)   # an early read would skip every row
    side.wait_stream(torch.cuda.current_stream())
    busy_current_stream()
    mb.mi_apply_bitmask_inplace(d, dm, wl.vocab_size, idx64, wl.fill_value, stream=side)
    torch.cuda.synchronize()
    assert np.array_equal(d.view(torch.int16).cpu().numpy().view(np.uint16), want)

    say("[gpu] side stream: out of place, int64 device indices, output allocated by the binding")
    d2 = bf16_bits_to_device(wl.logits)
    want_out = oracle.apply_out(wl.logits, wl.mask, wl.dtype, wl.vocab_size, list(wl.indices), wl.fill_value)
    torch.cuda.synchronize()
    poison_cache(idx64.numel(), torch.int32, -1)
    side.wait_stream(torch.cuda.current_stream())
    busy_current_stream()
    out = mb.mi_apply_bitmask_out(d2, dm, None, wl.vocab_size, idx64, wl.fill_value, stream=side)
    side.synchronize()
    torch.cuda.synchronize()
    assert np.array_equal(out.view(torch.int16).cpu().numpy().view(np.uint16), want_out)


def test_rows_bool_gate_and_report_on_side_stream():
    say("[gpu] side stream: bool gate, report allocated by the binding")
    rng = np.random.default_rng(31)
    wl = workloads.mixed_bf16(rows=48, vocab=5000, col_pad=0, word_pad=0, n_indices=0)
    wl.mask[5] = 0                         # an unsatisfiable row
    gate = rng.random(wl.rows) < 0.6
    gate[5] = True
    want = wl.logits.copy()
    oracle.apply_inplace(want, wl.mask, wl.dtype, wl.vocab_size, np.flatnonzero(gate).tolist(), wl.fill_value)
    want_any = oracle.apply_rows(wl.logits.copy(), wl.mask, wl.dtype, wl.vocab_size, gate.astype(np.int8),
                                 wl.fill_value)[1]
    d = bf16_bits_to_device(wl.logits)
    dm = torch.from_numpy(wl.mask).to("cuda")
    dg = torch.from_numpy(gate).to("cuda")           # bool: the binding casts it to int8
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    poison_cache(wl.rows, torch.int8, 0)             # an early read would gate every row off
    side.wait_stream(torch.cuda.current_stream())
    busy_current_stream()
    rep = mb.mi_apply_bitmask_rows(d, dm, dg, wl.vocab_size, wl.fill_value, report=True, stream=side)
    side.synchronize()
    torch.cuda.synchronize()
    assert np.array_equal(d.view(torch.int16).cpu().numpy().view(np.uint16), want)
    assert np.array_equal(rep.cpu().numpy(), np.asarray(want_any, dtype=np.uint8))


@pytest.mark.parametrize("workspace", ["auto", None])
def test_sampler_float64_params_on_side_stream(workspace):
    say(f"[gpu] side stream: float64 / int64 per-row sampler parameters, workspace={workspace}")
    rng = np.random.default_rng(32)
    wl = workloads.mixed_bf16(rows=16, vocab=20000, col_pad=0, word_pad=0, n_indices=0)
    d = bf16_bits_to_device(wl.logits)
    dm = torch.from_numpy(wl.mask).to("cuda")
    temp = torch.from_numpy(rng.uniform(0.5, 1.5, wl.rows)).to("cuda")                # float64
    top_k = torch.from_numpy(rng.integers(1, 200, wl.rows).astype(np.int64)).to("cuda")
    top_p = torch.from_numpy(rng.uniform(0.5, 0.95, wl.rows)).to("cuda")
    kw = dict(temperature=temp, top_k=top_k, top_p=top_p, seed=11, offset=3, workspace=workspace)
    want = mb.mi_apply_bitmask_sample(d, dm, wl.vocab_size, **kw).cpu()
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    poison_cache(wl.rows, torch.float32, 0.0)   # temperature 0: greedy rows
    poison_cache(wl.rows, torch.int32, 0)
    side.wait_stream(torch.cuda.current_stream())
    busy_current_stream()
    got = mb.mi_apply_bitmask_sample(d, dm, wl.vocab_size, stream=side, **kw)
    side.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(got.cpu(), want)
