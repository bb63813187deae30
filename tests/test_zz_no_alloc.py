"""The sampler entry point that allocates nothing, against the one that takes a workspace.

mi_apply_bitmask_sample_noalloc keeps the split path's workspace in a device
array of the library (32 rows' worth) instead of a caller's buffer.  Through
the C ABI, its tokens must equal mi_apply_bitmask_sample_ws's (given a
workspace it allocated) exactly: the same cut from the same counts, the same
Gumbel keys.  Two calls in a row, the second smaller, so the second runs on
what the first left in the array; then batches that need no workspace (the
split path takes at most 32 rows, which the array holds) run as before, and
large filtered batches keep their heavy-rows-first flags in the array.
"""

import sys

import numpy as np
import pytest

import workloads
import packed_logit_bitmask_amd as mb

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu-marked tests need an MI355X")
    mb.load_library()


def case(seed, dtype, rows, vocab, density=0.3):
    rng = np.random.default_rng(seed)
    vals = rng.standard_normal((rows, vocab)).astype(np.float32) * 2.0
    if dtype == "bfloat16":
        x = torch.from_numpy(vals).to("cuda").to(torch.bfloat16)
    else:
        x = torch.from_numpy(vals).to("cuda").to(torch.float16)
    mask = workloads.pack_allowed(rng.random((rows, vocab)) < density, (vocab + 31) // 32, rng)
    return x, torch.from_numpy(mask).to("cuda"), rng


def both(x, m, **kw):
    """Tokens from the workspace entry point and from the no-alloc one."""
    rows = x.shape[0]
    need = mb.sample_workspace_bytes(x.dtype, rows, x.shape[1])
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    a = mb.mi_apply_bitmask_sample(x, m, workspace=ws, **kw)
    out = torch.full((rows,), -7, dtype=torch.int64, device="cuda")
    b = mb.mi_apply_bitmask_sample_noalloc(x, m, out=out, **kw)
    torch.cuda.synchronize()
    assert b is out
    return need, a.cpu(), b.cpu()


def test_noalloc_matches_workspace_twice_second_smaller():
    say("[gpu] no-alloc sampler: 32 bf16 rows x 20000, then 8 fp16 rows x 12000")
    x, m, rng = case(1, "bfloat16", 32, 20000)
    temp = torch.from_numpy(rng.uniform(0.5, 1.5, 32).astype(np.float32)).to("cuda")
    top_k = torch.from_numpy(rng.integers(1, 300, 32).astype(np.int32)).to("cuda")
    need, a, b = both(x, m, temperature=temp, top_k=top_k, top_p=0.9, seed=3, offset=1)
    assert need > 0, "this batch must take the split path"
    assert torch.equal(a, b)
    assert (a >= 0).all()

    x, m, rng = case(2, "float16", 8, 12000)
    need, a, b = both(x, m, temperature=0.8, top_p=0.7, min_p=0.02, seed=4, offset=9)
    assert need > 0
    assert torch.equal(a, b)

    say("[gpu] no-alloc sampler: 20 rows, min-p only, after the calls above")
    x, m, rng = case(3, "bfloat16", 20, 9000)
    need, a, b = both(x, m, temperature=1.2, min_p=0.05, seed=5, offset=2)
    assert torch.equal(a, b)


def test_noalloc_batches_without_workspace():
    say("[gpu] no-alloc sampler: 40 filtered rows, past the split path, need no scratch")
    x, m, _ = case(4, "bfloat16", 40, 9000)
    need, a, b = both(x, m, temperature=1.0, top_k=40, seed=10)
    assert need == 0 and torch.equal(a, b)
    assert (a >= 0).all()
    say("[gpu] no-alloc sampler: batches that need no scratch")
    # unfiltered rows need no workspace at any batch size
    need, a, b = both(x, m, temperature=1.0, seed=6)
    assert torch.equal(a, b)
    # more rows than the split path takes, and fp32 rows, run one block per row
    x, m, _ = case(5, "float16", 100, 9000)
    need, a, b = both(x, m, temperature=1.0, top_p=0.8, seed=7)
    assert need == 0 and torch.equal(a, b)
    xf = x.float()
    need, a, b = both(xf, m, temperature=1.0, top_k=20, seed=8)
    assert need == 0 and torch.equal(a, b)
    # greedy rows
    x, m, _ = case(6, "bfloat16", 16, 9000)
    need, a, b = both(x, m, temperature=0.0, top_k=5)
    assert torch.equal(a, b)


def test_noalloc_orders_large_batches():
    # more filtered 16-bit rows than compute units: the dense rows go first,
    # their flags in the scratch; two calls in a row, the second smaller
    for seed, dtype, rows in ((7, "float16", 1024), (8, "bfloat16", 300)):
        say(f"[gpu] no-alloc sampler: {rows} {dtype} rows x 20000, top-p, heavy rows first")
        x, m, _ = case(seed, dtype, rows, 20000)
        dense = torch.rand(rows, device="cuda") < 0.3
        m[dense] = -1                                   # all allowed: dense rows among sparse ones
        need, a, b = both(x, m, temperature=1.0, top_p=0.9, min_p=0.02, seed=seed)
        assert need > 0 and torch.equal(a, b)
        assert (a >= 0).all()
