"""GPU parity of the fused apply + sampler against the sampler oracle.

Exact where the decision is exact: greedy picks (integer comparisons on the
same values) and rows with no candidate.  For draws, the GPU works in
binary32 and the oracle in binary64, so a draw may legitimately differ where
two Gumbel keys, or a token's probability and a filter's cutoff, agree to
within float rounding; the oracle reports those cases as a candidate set
(margin 1e-4) and the GPU token must be in it.  The number of draws that
match the oracle's own draw exactly is checked too.  The draw distribution
is checked with a chi-square test against the renormalised filtered softmax.
"""

import math
import sys

import numpy as np
import pytest

from oracle import sampler as S
import workloads
import packed_logit_bitmask_amd as mb

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TORCH = {"float32": (np.int32, torch.float32), "float16": (np.int16, torch.float16),
         "bfloat16": (np.int16, torch.bfloat16)}
MARGIN = 1e-4


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu-marked tests need an MI355X")
    mb.load_library()


def values64(bits, dtype):
    if dtype == "float32":
        return bits.view(np.float32).astype(np.float64)
    if dtype == "float16":
        return bits.view(np.float16).astype(np.float64)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def dev_logits(bits, dtype):
    ndt, tdt = TORCH[dtype]
    return torch.from_numpy(np.ascontiguousarray(bits).view(ndt)).to("cuda").view(tdt)


def per_row(v, i):
    return v[i] if isinstance(v, np.ndarray) else v


def check_rows(bits, dtype, mask, vocab, T, k, p, m, seed, offset, rows=None, min_exact=0.98, workspace="auto"):
    """Sample on the GPU and check every row against the oracle; returns the tokens.
    workspace: as for mi_apply_bitmask_sample ("auto" splits a small batch of
    filtered 16-bit rows over several blocks; None keeps one block per row)."""
    R, cols = bits.shape
    dl = dev_logits(bits, dtype)
    dm = None if mask is None else torch.from_numpy(np.ascontiguousarray(mask)).to("cuda")
    targs = {}
    for name, v, td in (("temperature", T, torch.float32), ("top_k", k, torch.int32),
                        ("top_p", p, torch.float32), ("min_p", m, torch.float32)):
        targs[name] = torch.from_numpy(v).to("cuda", td) if isinstance(v, np.ndarray) else v
    tok = mb.mi_apply_bitmask_sample(dl, dm, vocab, seed=seed, offset=offset, workspace=workspace,
                                     **targs).cpu().numpy()
    V = cols if vocab is None and mask is None else (vocab if vocab is not None else
                                                     min(cols, 32 * mask.shape[1]))
    vals = values64(bits, dtype)
    exact = 0
    for r in (range(R) if rows is None else rows):
        allowed = S.allowed_tokens(None if mask is None else mask[r], V, cols)
        want, det = S.sample_row(vals[r], allowed, float(per_row(T, r)), int(per_row(k, r)), float(per_row(p, r)),
                                 float(per_row(m, r)), seed, offset, r, margin=MARGIN)
        assert tok[r] in det["candidates"], (r, tok[r], want, sorted(det["candidates"])[:5])
        if tok[r] >= 0:
            assert allowed[tok[r]], (r, tok[r])
        exact += int(tok[r] == want)
    n = R if rows is None else len(rows)
    assert exact >= min_exact * n, f"only {exact}/{n} draws equal the oracle's"
    return tok


def random_logits(rng, dtype, R, cols, sigma=2.0, ties=False):
    """N(0, sigma) logits as dtype bit patterns; with ties, rounded to halves (many equal values)."""
    x = rng.standard_normal((R, cols)).astype(np.float32) * np.float32(sigma)
    if ties:
        x = np.round(x * 2) / 2
    if dtype == "float32":
        return x.view(np.uint32)
    if dtype == "float16":
        return x.astype(np.float16).view(np.uint16)
    b = x.view(np.uint32)
    return ((b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


@pytest.mark.parametrize("dtype", ["float32", "float16", "bfloat16"])
def test_greedy_exact_with_ties_and_masks(dtype):
    rng = np.random.default_rng(1)
    R, cols = 40, 3000
    bits = random_logits(rng, dtype, R, cols, ties=True)
    mask = workloads.pack_allowed(rng.random((R, cols)) < 0.3, (cols + 31) // 32, rng)
    mask[5] = 0                                       # an unsatisfiable row
    say(f"[gpu] sampler greedy {dtype}")
    tok = check_rows(bits, dtype, mask, None, 0.0, 0, 1.0, 0.0, 1, 2, min_exact=1.0)
    assert tok[5] == -1
    check_rows(bits, dtype, None, 2500, -1.0, 5, 0.5, 0.1, 1, 2, min_exact=1.0)


@pytest.mark.parametrize("T,k,p,m", [(1.0, 0, 1.0, 0.0), (0.7, 40, 1.0, 0.0), (1.2, 0, 0.9, 0.0),
                                      (1.0, 0, 1.0, 0.02), (0.8, 100, 0.95, 0.01), (1.5, 1, 1.0, 0.0),
                                      (1.0, 5000, 0.3, 0.0),
                                      # edges: p = 0 and p < 0 keep only the max (and its ties); min_p = 1
                                      # likewise; k above the vocab keeps everything; a tiny temperature
                                      (1.0, 0, 0.0, 0.0), (1.0, 0, -0.5, 0.0), (1.0, 0, 1.0, 1.0),
                                      (1.0, 100000, 1.0, 0.0), (1e-3, 0, 1.0, 0.0), (math.nan, 0, 0.9, 0.0),
                                      # min_p above 1 keeps the max; an infinite temperature keeps everything
                                      (1.0, 0, 1.0, 1.5), (math.inf, 5, 0.5, 0.2)])
def test_draws_match_oracle(T, k, p, m):
    rng = np.random.default_rng(2)
    R, cols = 48, 4100
    dtype = "bfloat16"
    bits = random_logits(rng, dtype, R, cols)
    mask = workloads.pack_allowed(rng.random((R, cols)) < rng.uniform(0.05, 0.9, (R, 1)), 129, rng)
    say(f"[gpu] sampler draws T={T} k={k} p={p} m={m}")
    check_rows(bits, dtype, mask, 4100, T, k, p, m, seed=11, offset=3)


def test_per_row_parameters_verify_shape():
    rng = np.random.default_rng(3)
    wl = workloads.verify_fp16()
    R = wl.rows
    T = rng.choice([0.0, 0.5, 1.0, 1.3], R).astype(np.float32)
    k = rng.choice([0, 1, 20, 500], R).astype(np.int32)
    p = rng.choice([1.0, 0.9, 0.6], R).astype(np.float32)
    m = rng.choice([0.0, 0.05], R).astype(np.float32)
    say("[gpu] sampler per-row parameters on the [1024, 32000] fp16 verify shape")
    tok = check_rows(wl.logits, "float16", wl.mask, None, T, k, p, m, seed=7, offset=9)   # every row
    zero_rows = [r for r in range(R) if not (wl.mask[r] != 0).any()]
    assert all(tok[r] == -1 for r in zero_rows) and zero_rows


def test_full_size_mixed_bf16_with_mask():
    wl = workloads.mixed_bf16()
    say("[gpu] sampler on the [256, 128256] bf16 shape, vocab 128000, masked")
    check_rows(wl.logits, "bfloat16", wl.mask, 128000, 0.8, 0, 0.9, 0.0, seed=123, offset=1)   # every row
    check_rows(wl.logits, "bfloat16", wl.mask, 128000, 1.0, 50, 1.0, 0.0, seed=123, offset=2)


def test_large_vocab_fp32():
    wl = workloads.large_fp32(rows=8)
    say("[gpu] sampler on fp32 rows of 262144 (vocab 262100)")
    check_rows(wl.logits, "float32", wl.mask, 262100, 1.0, 0, 0.95, 0.001, seed=5, offset=5)


def test_determinism_and_offset():
    rng = np.random.default_rng(4)
    bits = random_logits(rng, "float32", 256, 2000)
    dl = dev_logits(bits, "float32")
    a = mb.mi_apply_bitmask_sample(dl, seed=9, offset=4, top_p=0.95).cpu().numpy()
    b = mb.mi_apply_bitmask_sample(dl, seed=9, offset=4, top_p=0.95).cpu().numpy()
    c = mb.mi_apply_bitmask_sample(dl, seed=9, offset=5, top_p=0.95).cpu().numpy()
    d = mb.mi_apply_bitmask_sample(dl, seed=10, offset=4, top_p=0.95).cpu().numpy()
    assert np.array_equal(a, b)
    assert (a != c).mean() > 0.7 and (a != d).mean() > 0.7


def test_distribution_chi_square():
    rng = np.random.default_rng(5)
    z = (rng.standard_normal(64) * 2.0).astype(np.float32)
    allowed = np.ones(64, bool)
    allowed[[7, 30, 31]] = False
    mask_row = workloads.pack_allowed(allowed[None, :], 2, None, garbage=False)
    R = 4096
    bits = np.repeat(z.view(np.uint32)[None, :], R, axis=0)
    mask = np.repeat(mask_row, R, axis=0)
    T, k, p, m = 0.9, 20, 0.95, 0.01
    dl = dev_logits(bits, "float32")
    dm = torch.from_numpy(mask).to("cuda")
    toks = np.concatenate([mb.mi_apply_bitmask_sample(dl, dm, temperature=T, top_k=k, top_p=p, min_p=m, seed=3,
                                                      offset=o).cpu().numpy() for o in range(5)])
    probs = S.filtered_probs(z.astype(np.float64), allowed, T, k, p, m)
    counts = np.bincount(toks, minlength=64)
    assert counts[probs == 0].sum() == 0
    exp = probs * toks.size
    big = exp >= 5
    stat = (((counts[big] - exp[big]) ** 2) / exp[big]).sum()
    dof = int(big.sum()) - 1
    zscore = ((stat / dof) ** (1 / 3) - (1 - 2 / (9 * dof))) / math.sqrt(2 / (9 * dof))
    say(f"[gpu] chi-square {stat:.1f} on {dof} dof (z = {zscore:.2f})")
    assert zscore < 4.75
    assert np.abs(counts / toks.size - probs).max() < 0.01


@pytest.mark.parametrize("dtype", ["float32", "float16", "bfloat16"])
def test_signed_zero_ties_at_the_cut(dtype):
    """A top-k cut that falls on zero keeps +0 and -0 alike (they compare equal)."""
    R, cols = 64, 96
    x = np.full(cols, -3.0, np.float32)
    x[0] = 2.0
    x[1] = 0.0
    x[2:22] = -0.0                    # twenty negative zeros after one positive zero
    bits = np.repeat(x[None, :], R, axis=0)
    if dtype == "float32":
        bits = bits.view(np.uint32)
    elif dtype == "float16":
        bits = bits.astype(np.float16).view(np.uint16)
    else:
        bits = (bits.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    say(f"[gpu] sampler signed-zero ties {dtype}")
    tok = check_rows(bits, dtype, None, None, 1.0, 2, 1.0, 0.0, seed=21, offset=0)
    assert ((tok >= 2) & (tok < 22)).sum() > R // 4, "negative zeros were cut"
    assert tok.max() < 22
    tok = check_rows(bits, dtype, None, None, 1.0, 0, 0.3, 0.0, seed=22, offset=1)
    assert tok.max() < 22


@pytest.mark.parametrize("dtype", ["float32", "float16", "bfloat16"])
def test_misaligned_rows_and_ragged_tail(dtype):
    """Rows that start off a 16-byte boundary (odd row length, and a view one
    element into the buffer) and a vocab size that leaves a partial last
    group of 8 tokens."""
    rng = np.random.default_rng(8)
    R, cols, V = 24, 4099, 4093
    full = random_logits(rng, dtype, R, cols + 1)
    mask = workloads.pack_allowed(rng.random((R, cols)) < 0.4, (cols + 31) // 32, rng)
    ndt, tdt = TORCH[dtype]
    dl = torch.from_numpy(np.ascontiguousarray(full).view(ndt)).to("cuda").view(tdt)[:, 1:]
    assert dl.data_ptr() % 16 != 0
    dm = torch.from_numpy(mask).to("cuda")
    bits = np.ascontiguousarray(full[:, 1:])
    vals = values64(bits, dtype)
    say(f"[gpu] sampler misaligned rows {dtype}")
    for (T, k, p, m) in ((0.0, 0, 1.0, 0.0), (1.0, 0, 1.0, 0.0), (0.9, 30, 1.0, 0.0), (1.1, 0, 0.8, 0.02)):
        tok = mb.mi_apply_bitmask_sample(dl, dm, V, temperature=T, top_k=k, top_p=p, min_p=m, seed=4,
                                         offset=2).cpu().numpy()
        exact = 0
        for r in range(R):
            allowed = S.allowed_tokens(mask[r], V, cols)
            want, det = S.sample_row(vals[r], allowed, T, k, p, m, 4, 2, r, margin=MARGIN)
            assert tok[r] in det["candidates"], (T, k, p, m, r, tok[r], want)
            exact += int(tok[r] == want)
        assert exact >= R - 1
        # a contiguous copy (other row alignments) gives the same tokens
        again = mb.mi_apply_bitmask_sample(dl.contiguous(), dm, V, temperature=T, top_k=k, top_p=p, min_p=m,
                                           seed=4, offset=2).cpu().numpy()
        assert np.array_equal(tok, again)


@pytest.mark.parametrize("T,k,p,m", [(0.0, 0, 1.0, 0.0), (1.0, 0, 1.0, 0.0), (1.0, 7, 1.0, 0.0),
                                      (1.0, 0, 0.9, 0.0), (1.0, 0, 1.0, 0.1), (0.7, 7, 0.9, 0.1)])
def test_rows_without_candidates_draw_minus_one(T, k, p, m):
    """Every mode (some skip the max pass) returns -1 for a row with nothing
    allowed: an all-zero mask row, or allowed tokens whose logits are all
    -inf; a single allowed token is always drawn."""
    rng = np.random.default_rng(9)
    R, cols = 16, 777
    x = rng.standard_normal((R, cols)).astype(np.float32)
    allowed = rng.random((R, cols)) < 0.5
    allowed[3] = False
    x[7, allowed[7]] = -np.inf
    allowed[11] = False
    allowed[11, 500] = True
    mask = workloads.pack_allowed(allowed, (cols + 31) // 32, rng)
    say(f"[gpu] sampler empty rows T={T} k={k} p={p} m={m}")
    tok = check_rows(x.view(np.uint32), "float32", mask, None, T, k, p, m, seed=2, offset=5, min_exact=1.0)
    assert tok[3] == -1 and tok[7] == -1 and tok[11] == 500


def test_graph_replay_matches_eager():
    """The sampler captured in a HIP graph (several offsets, a per-row
    temperature array) replays to the eager tokens, replay after replay,
    with other GPU work and synchronisations in between."""
    rng = np.random.default_rng(10)
    R, cols = 64, 5000
    bits = random_logits(rng, "bfloat16", R, cols)
    mask = workloads.pack_allowed(rng.random((R, cols)) < 0.3, (cols + 31) // 32, rng)
    dl = dev_logits(bits, "bfloat16")
    dm = torch.from_numpy(mask).to("cuda")
    temp = torch.from_numpy(rng.uniform(0.5, 1.5, R).astype(np.float32)).to("cuda")
    modes = [dict(top_k=20), dict(top_p=0.8), dict(min_p=0.05), dict()]
    outs = [torch.empty(R, dtype=torch.int64, device="cuda") for _ in modes]
    want = [mb.mi_apply_bitmask_sample(dl, dm, 4990, temperature=temp, seed=5, offset=k, **kw).cpu()
            for k, kw in enumerate(modes)]
    say("[gpu] sampler graph capture")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for k, kw in enumerate(modes):
                mb.mi_apply_bitmask_sample(dl, dm, 4990, temperature=temp, seed=5, offset=k, out=outs[k], **kw)
    torch.cuda.synchronize()
    for rep in range(3):
        for o in outs:
            o.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        for k in range(len(modes)):
            assert torch.equal(outs[k].cpu(), want[k]), (rep, modes[k])
        (dl.float() * 2).sum().item()     # unrelated eager work between replays
    del g


@pytest.mark.parametrize("dtype,filters", [("float32", True), ("bfloat16", True), ("float16", False)])
def test_many_rows_variant(dtype, filters):
    """More than 256 rows: fp32 rows, and 16-bit rows without top-k or top-p,
    take the 256-thread variant; 16-bit rows that may filter take 512-thread
    blocks with the 8-bit-counter key histogram.  Per-row parameters, a ragged
    vocab tail and a few rows with nothing allowed."""
    rng = np.random.default_rng(11)
    R, cols, V = 300, 2051, 2045
    bits = random_logits(rng, dtype, R, cols)
    allowed = rng.random((R, cols)) < rng.uniform(0.02, 0.8, (R, 1))
    allowed[[4, 150, 299]] = False
    mask = workloads.pack_allowed(allowed, (cols + 31) // 32, rng)
    T = rng.choice([0.0, 0.6, 1.0, 1.4], R).astype(np.float32)
    k = rng.choice([0, 1, 10, 300] if filters else [0], R).astype(np.int32)
    p = rng.choice([1.0, 0.95, 0.5] if filters else [1.0], R).astype(np.float32)
    m = rng.choice([0.0, 0.02], R).astype(np.float32)
    say(f"[gpu] sampler 300 rows {dtype} filters={filters}")
    tok = check_rows(bits, dtype, mask, V, T, k, p, m, seed=13, offset=77)
    assert tok[4] == -1 and tok[150] == -1 and tok[299] == -1


@pytest.mark.parametrize("dtype", ["float16", "bfloat16"])
def test_key_holding_65536_tokens(dtype):
    """16-bit rows count their tokens per key in 16 bits; a key holding 65536
    or more candidates would wrap, and the row then takes the radix search.
    Rows with 65535 (no wrap), 65536 and 66000 copies of one value among
    random logits, and a row without copies, under top-k (a cut above the
    copies, and one that keeps them all) and top-p."""
    rng = np.random.default_rng(19)
    R, cols = 4, 70003
    bits = random_logits(rng, dtype, R, cols)
    one = {"float16": 0x3400, "bfloat16": 0x3E80}[dtype]          # 0.25
    bits[bits == one] = one + 1                                   # only the planted copies hold 0.25
    for r, copies in enumerate((65535, 65536, 66000, 0)):
        bits[r, rng.choice(cols, copies, replace=False)] = one
    for ws in (None, "auto"):    # one block per row (16-bit LDS counters), and split (32-bit counts)
        say(f"[gpu] sampler keys holding 65536 tokens {dtype} workspace={ws}")
        for (T, k, p, seed) in ((1.0, 10, 1.0, 1), (1.0, 2000, 1.0, 2), (0.9, 0, 0.6, 3), (1.0, 50, 0.9, 4)):
            check_rows(bits, dtype, None, None, T, k, p, 0.0, seed=seed, offset=0, min_exact=0.75, workspace=ws)


@pytest.mark.parametrize("dtype", ["float16", "bfloat16"])
def test_many_rows_keys_holding_256_tokens(dtype):
    """With more rows than compute units, filtered 16-bit rows count their
    keys in 8 bits; a key holding 256 or more candidates would wrap, and the
    row then takes the radix search.  300 rows, five of them with 255 (no
    wrap), 256, 257, 1000 and 3000 copies of one value among random logits,
    under top-k (a cut above the copies, and one that keeps them), top-p and
    all three filters, with a mask on every row."""
    rng = np.random.default_rng(43)
    R, cols = 300, 4099
    bits = random_logits(rng, dtype, R, cols)
    one = {"float16": 0x3400, "bfloat16": 0x3E80}[dtype]          # 0.25
    bits[bits == one] = one + 1                                   # only the planted copies hold 0.25
    for r, copies in enumerate((255, 256, 257, 1000, 3000)):
        bits[r, rng.choice(cols, copies, replace=False)] = one
    allowed = rng.random((R, cols)) < 0.9
    for r, copies in enumerate((255, 256, 257, 1000, 3000)):
        allowed[r, bits[r] == one] = True                         # every copy is a candidate
    mask = workloads.pack_allowed(allowed, (cols + 31) // 32, rng)
    say(f"[gpu] sampler 300 rows, keys holding 256 tokens {dtype}")
    for (T, k, p, m, seed) in ((1.0, 10, 1.0, 0.0, 1), (1.0, 2500, 1.0, 0.0, 2), (0.9, 0, 0.6, 0.0, 3),
                               (1.0, 50, 0.9, 0.05, 4)):
        check_rows(bits, dtype, mask, None, T, k, p, m, seed=seed, offset=0, min_exact=0.9)


@pytest.mark.parametrize("dtype", ["float16", "bfloat16"])
def test_fuzz_filtered_16bit_many_rows(dtype):
    """Seeded random batches of 257 to 700 rows (the 8-bit-counter histogram
    in 512-thread blocks): shapes, masks, value spreads (heavy ties among
    them, which may wrap a counter), and per-row filter settings."""
    rng = np.random.default_rng(47 if dtype == "float16" else 53)
    for case in range(4):
        R = int(rng.integers(257, 700))
        cols = int(rng.integers(1, 3000))
        ties = bool(rng.integers(0, 2))
        bits = random_logits(rng, dtype, R, cols, sigma=float(rng.choice([0.3, 2.0, 8.0])), ties=ties)
        density = rng.uniform(0.0, 1.0, (R, 1))
        mask = workloads.pack_allowed(rng.random((R, cols)) < density, (cols + 31) // 32 + int(rng.integers(0, 2)), rng)
        V = int(rng.integers(1, cols + 1))
        T = rng.choice([0.0, 0.5, 1.0, 1.7], R).astype(np.float32)
        k = rng.choice([0, 1, 5, 50, 400, 10000], R).astype(np.int32)
        p = rng.choice([1.0, 0.99, 0.9, 0.5, 0.1], R).astype(np.float32)
        m = rng.choice([0.0, 0.0, 0.05], R).astype(np.float32)
        say(f"[gpu] sampler fuzz many rows {dtype} case {case}: R={R} cols={cols} V={V} ties={ties}")
        check_rows(bits, dtype, mask, V, T, k, p, m, seed=200 + case, offset=case, min_exact=0.9)


@pytest.mark.parametrize("dtype,R", [("float16", 1100), ("bfloat16", 1101), ("float32", 1030)])
def test_tokens_independent_of_batch_size(dtype, R):
    """The generator is keyed by the row, so a row's token does not depend on
    how many rows share the launch, although the kernel does: 16-bit rows
    take 1024-thread blocks with 16-bit counters up to 256 rows and 512-thread
    blocks with 8-bit counters beyond; fp32 rows the coarse-bucket cut in
    1024-thread blocks up to 256 rows and the radix search in 256-thread
    blocks beyond.  Rows of mixed densities (all allowed, none, sparse) and
    per-row filters; the first 256 and 520 rows of the batch must draw the
    same tokens as the whole batch, and a sample of rows is checked against
    the oracle."""
    rng = np.random.default_rng(71 + R)
    cols = 3000 if dtype != "float32" else 700
    bits = random_logits(rng, dtype, R, cols)
    kind = rng.choice(4, R, p=[0.2, 0.05, 0.5, 0.25])           # all allowed, none, sparse, medium
    dens = np.choose(kind, [1.0, 0.0, 0.05, 0.5])[:, None]
    allowed = rng.random((R, cols)) < dens
    mask = workloads.pack_allowed(allowed, (cols + 31) // 32, rng)
    T = rng.choice([0.6, 1.0, 1.3], R).astype(np.float32)
    k = rng.choice([0, 5, 60], R).astype(np.int32)
    p = rng.choice([1.0, 0.9, 0.5], R).astype(np.float32)
    m = rng.choice([0.0, 0.03], R).astype(np.float32)
    say(f"[gpu] sampler tokens independent of batch size {dtype} R={R}")
    tok = check_rows(bits, dtype, mask, None, T, k, p, m, seed=73, offset=5, rows=list(range(0, R, 7)),
                     min_exact=0.9)
    assert (tok[kind == 1] == -1).all() and (tok[kind != 1] >= 0).all()
    for n in (256, 520):
        part = check_rows(bits[:n], dtype, mask[:n], None, T[:n], k[:n], p[:n], m[:n], seed=73, offset=5,
                          rows=[], min_exact=0.0)
        assert (part == tok[:n]).all(), f"{int((part != tok[:n]).sum())} of the first {n} rows differ"


@pytest.mark.parametrize("dtype,V", [("float16", 20003), ("bfloat16", 20003), ("bfloat16", 50001)])
def test_sparse_rows_listed_search(dtype, V):
    """Filtered 16-bit rows whose mask allows at most 4096 tokens take their
    cuts from a list of the candidates instead of the 65536-key histogram.
    Rows allowing 0, 1, 7, 4095, 4096 (listed) and 4097 (histogram) tokens;
    2000 allowed tokens all in one wave's groups
    (its list region overflows: histogram); ties among the candidates, -0
    and +0, NaN and infinities among the allowed tokens, and a row whose
    allowed tokens are all NaN or infinite (no candidate: -1); k beyond the
    candidates, p = 0, min-p; a misaligned row pitch and a ragged vocab.
    Every row against the oracle; the first 256 rows against the same rows
    drawn as a batch of 256 (1024-thread blocks); and every row against the
    histogram search on the same candidates (no mask, disallowed logits at
    -inf): the same tokens.  A row of 50001 tokens is read in two batches
    of groups per thread, one of 20003 in one."""
    rng = np.random.default_rng((97 if dtype == "float16" else 101) + V)
    R, cols = 300, V + 8
    bits = random_logits(rng, dtype, R, cols, sigma=1.5)
    allowed = np.zeros((R, cols), bool)
    counts = [0, 1, 7, 4095, 4096, 4097, 60, 2000, 300, 4096]
    for r in range(R):
        n = counts[r % len(counts)] if r < 200 else int(rng.integers(0, 3000))
        allowed[r, rng.choice(V, min(n, V), replace=False)] = True
    group = np.arange(cols) // 8
    wave0 = np.flatnonzero(((group % 512) < 64) & (np.arange(cols) < V))
    for r in (10, 11):                            # crowd wave 0's region (1024 entries)
        allowed[r] = False
        allowed[r, rng.choice(wave0, 2000, replace=False)] = True
    # ties, signed zeros and non-finite values among the candidates
    zero = {"float16": (0x0000, 0x8000), "bfloat16": (0x0000, 0x8000)}[dtype]
    inf, nan = {"float16": (0x7C00, 0x7E00), "bfloat16": (0x7F80, 0x7FC0)}[dtype]
    for r in range(0, R, 3):
        idx = np.flatnonzero(allowed[r])
        if idx.size >= 8:
            bits[r, idx[:3]] = zero[0]
            bits[r, idx[3:5]] = zero[1]
            bits[r, idx[5]] = nan
            bits[r, idx[6]] = inf
            bits[r, idx[7]] = inf | 0x8000
            bits[r, idx[8:12]] = bits[r, idx[12]] if idx.size > 12 else bits[r, idx[8]]
    # a row whose allowed tokens are all NaN or infinite: no candidate
    allowed[13] = False
    only = rng.choice(V, 6, replace=False)
    allowed[13, only] = True
    bits[13, only] = [nan, inf, inf | 0x8000, nan, inf, nan]
    mask = workloads.pack_allowed(allowed, (cols + 31) // 32 + 1, rng)
    pitch = cols + 3                                # rows start off a 16-byte boundary
    padded = np.zeros((R, pitch), bits.dtype)
    padded[:, :cols] = bits
    T = rng.choice([0.7, 1.0, 1.3], R).astype(np.float32)
    k = rng.choice([0, 1, 5, 100, 5000], R).astype(np.int32)
    p = rng.choice([1.0, 0.9, 0.5, 0.0], R).astype(np.float32)
    m = rng.choice([0.0, 0.0, 0.05], R).astype(np.float32)
    say(f"[gpu] sampler sparse rows listed search {dtype} V={V}")
    dl = dev_logits(padded, dtype)[:, :cols]
    dm = torch.from_numpy(np.ascontiguousarray(mask)).to("cuda")
    targs = dict(temperature=torch.from_numpy(T).cuda(), top_k=torch.from_numpy(k).cuda(),
                 top_p=torch.from_numpy(p).cuda(), min_p=torch.from_numpy(m).cuda())
    tok = mb.mi_apply_bitmask_sample(dl, dm, V, seed=103, offset=9, **targs).cpu().numpy()
    part = mb.mi_apply_bitmask_sample(dl[:256], dm[:256], V, seed=103, offset=9,
                                      **{n: v[:256] for n, v in targs.items()}).cpu().numpy()
    assert (part == tok[:256]).all(), f"{int((part != tok[:256]).sum())} of the first 256 rows differ"
    # the same candidates without a mask, every disallowed logit at -inf: the
    # histogram search (the list needs a mask), which must draw the same tokens
    hist_bits = padded.copy()
    hist_bits[:, :cols][~allowed] = {"float16": 0xFC00, "bfloat16": 0xFF80}[dtype]
    tok_h = mb.mi_apply_bitmask_sample(dev_logits(hist_bits, dtype)[:, :cols], None, V, seed=103, offset=9,
                                       **targs).cpu().numpy()
    assert (tok_h == tok).all(), f"{int((tok_h != tok).sum())} rows differ from the histogram search"
    vals = values64(bits, dtype)
    exact = 0
    for r in range(R):
        al = S.allowed_tokens(mask[r], V, cols)
        want, det = S.sample_row(vals[r], al, float(T[r]), int(k[r]), float(p[r]), float(m[r]), 103, 9, r,
                                 margin=MARGIN)
        assert tok[r] in det["candidates"], (r, tok[r], want)
        exact += int(tok[r] == want)
    assert exact >= 0.98 * R, f"only {exact}/{R} draws equal the oracle's"
    assert tok[0] == -1 and tok[13] == -1 and (tok[allowed[:, :V].sum(1) == 0] == -1).all()


@pytest.mark.parametrize("dtype", ["float16", "bfloat16"])
def test_sparse_long_rows_one_block_each(dtype):
    """Sparse rows longer than two batches of groups per thread of a 1024-thread
    block (140 001 tokens: the count and the listing each walk three batches)
    in a batch of 8 rows, one block per row (no workspace).  Rows allowing 0,
    3, 600, 4096 and 4097 tokens (the last through the histogram search);
    every row against the oracle and against the histogram search on the
    same candidates (no mask, disallowed logits at -inf): the same tokens."""
    rng = np.random.default_rng(107 if dtype == "float16" else 109)
    R, V = 8, 140001
    cols = V + 5
    bits = random_logits(rng, dtype, R, cols, sigma=1.5)
    allowed = np.zeros((R, cols), bool)
    for r, n in enumerate([0, 3, 600, 4096, 4097, 1500, 50, 4000]):
        allowed[r, rng.choice(V, n, replace=False)] = True
    mask = workloads.pack_allowed(allowed, (cols + 31) // 32, rng)
    T = rng.choice([0.7, 1.0, 1.3], R).astype(np.float32)
    k = np.array([5, 0, 100, 50, 50, 0, 2, 3000], np.int32)
    p = np.array([1.0, 0.9, 0.5, 0.9, 0.9, 0.3, 1.0, 0.95], np.float32)
    m = np.array([0.0, 0.0, 0.05, 0.0, 0.0, 0.02, 0.0, 0.0], np.float32)
    say(f"[gpu] sampler sparse long rows {dtype}")
    targs = dict(temperature=torch.from_numpy(T).cuda(), top_k=torch.from_numpy(k).cuda(),
                 top_p=torch.from_numpy(p).cuda(), min_p=torch.from_numpy(m).cuda())
    dm = torch.from_numpy(np.ascontiguousarray(mask)).to("cuda")
    tok = mb.mi_apply_bitmask_sample(dev_logits(bits, dtype), dm, V, seed=113, offset=4, workspace=None,
                                     **targs).cpu().numpy()
    hist_bits = bits.copy()
    hist_bits[~allowed] = {"float16": 0xFC00, "bfloat16": 0xFF80}[dtype]
    tok_h = mb.mi_apply_bitmask_sample(dev_logits(hist_bits, dtype), None, V, seed=113, offset=4, workspace=None,
                                       **targs).cpu().numpy()
    assert (tok_h == tok).all(), (tok, tok_h)
    vals = values64(bits, dtype)
    for r in range(R):
        al = S.allowed_tokens(mask[r], V, cols)
        want, det = S.sample_row(vals[r], al, float(T[r]), int(k[r]), float(p[r]), float(m[r]), 113, 4, r,
                                 margin=MARGIN)
        assert tok[r] in det["candidates"], (r, tok[r], want)
    assert tok[0] == -1 and (tok[1:] >= 0).all()


@pytest.mark.parametrize("dtype", ["float16", "bfloat16"])
def test_kept_tokens_crowding_one_wave_many_rows(dtype):
    """As the test above for 512-thread blocks (more rows than compute units):
    8 waves, each with a list region of 2048 entries.  6000 kept tokens all
    in wave 0's groups (groups g with g % 512 < 64) overflow its region, so
    the row takes the walk; the GPU draws every row, the oracle checks 12."""
    rng = np.random.default_rng(59)
    R, cols = 300, 60000
    x = rng.standard_normal((R, cols)).astype(np.float32) - np.float32(12.0)
    group = np.arange(cols) // 8
    x[:, (group % 512) < 64] += np.float32(16.0)       # wave 0's groups: 7504 tokens around +4
    if dtype == "float16":
        bits = x.astype(np.float16).view(np.uint16)
    else:
        b = x.view(np.uint32)
        bits = ((b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
    rows = list(range(0, R, 25))
    say(f"[gpu] sampler kept tokens crowding one wave, 300 rows {dtype}")
    check_rows(bits, dtype, None, None, 1.0, 6000, 1.0, 0.0, seed=61, offset=1, rows=rows, min_exact=0.75)
    check_rows(bits, dtype, None, None, 1.0, 0, 0.999, 0.0, seed=62, offset=2, rows=rows, min_exact=0.75)


def test_fp32_top_k_two_pass_cut():
    """fp32 rows with top-k alone: one coarse pass counts candidates per
    eighth of a binade, and the draw lists the bucket holding the k-th
    largest for an exact select.  Rows whose cut falls among 5000 distinct
    values that share one bucket (1 + i * 2^-21), next to random logits; k
    above, at and inside the crowded bucket; a row with ties at the cut; and
    with min-p and a mask.  Against the oracle."""
    rng = np.random.default_rng(107)
    R, cols = 6, 40000
    x = rng.standard_normal((R, cols)).astype(np.float32)
    x[x >= 1.0] -= np.float32(2.0)                                    # nothing random at or above 1
    for r in range(R):
        pos = rng.choice(cols, 5000, replace=False)
        x[r, pos] = np.float32(1.0) + np.arange(5000, dtype=np.float32) * np.float32(2.0 ** -21)
    x[5, rng.choice(cols, 300, replace=False)] = np.float32(1.0) + np.float32(2000 * 2.0 ** -21)  # ties at a cut
    bits = x.view(np.uint32)
    allowed = rng.random((R, cols)) < 0.9
    mask = workloads.pack_allowed(allowed, (cols + 31) // 32, rng)
    for (k, m, seed) in ((1, 0.0, 1), (10, 0.0, 2), (2500, 0.0, 3), (4600, 0.0, 4), (6000, 0.0, 5),
                         (3000, 0.02, 6), (40000, 0.0, 7)):
        say(f"[gpu] fp32 two-pass top-k k={k} min_p={m}")
        check_rows(bits, "float32", mask, None, 1.0, k, 1.0, m, seed=seed, offset=k, min_exact=0.9)
        check_rows(bits, "float32", None, None, 0.8, k, 1.0, m, seed=seed, offset=k + 1, min_exact=0.9)


def test_fp32_top_k_bucket_holding_65536_tokens():
    """A coarse bucket of an fp32 row holding 65535, 65536 or 66000
    candidates, more than the list holds: the row then takes the radix search
    over the whole row.  Distinct values inside the bucket, top-k cuts inside
    and above it."""
    rng = np.random.default_rng(109)
    R, cols = 3, 70003
    x = rng.standard_normal((R, cols)).astype(np.float32) - np.float32(3.0)
    x[x >= 1.0] = np.float32(0.5)
    for r, copies in enumerate((65535, 65536, 66000)):
        pos = rng.choice(cols, copies, replace=False)
        x[r, pos] = np.float32(1.0) + (np.arange(copies) % 4096).astype(np.float32) * np.float32(2.0 ** -20)
    bits = x.view(np.uint32)
    for (k, seed) in ((10, 1), (30000, 2), (65600, 3)):
        say(f"[gpu] fp32 bucket holding 65536 tokens k={k}")
        check_rows(bits, "float32", None, None, 1.0, k, 1.0, 0.0, seed=seed, offset=0, min_exact=0.9)


def crowded_fp32_rows(rng, R, cols, crowd, shift=-2.0):
    """N(0,1) + shift logits with `crowd` distinct values 1 + i * 2^-21 (one
    coarse bucket, an eighth of the binade [1, 2)) placed at random, so most
    of the softmax mass sits inside that bucket."""
    x = rng.standard_normal((R, cols)).astype(np.float32) + np.float32(shift)
    x[x >= 1.0] = np.float32(0.75)
    for r in range(R):
        pos = rng.choice(cols, crowd, replace=False)
        x[r, pos] = np.float32(1.0) + np.arange(crowd, dtype=np.float32) * np.float32(2.0 ** -21)
    return x


@pytest.mark.parametrize("k,p,m", [(0, 0.5, 0.0), (0, 0.1, 0.0), (0, 0.9, 0.0), (0, 0.999, 0.0),
                                   (2500, 0.9, 0.0), (6000, 0.5, 0.0), (2500, 0.5, 0.0), (2500, 0.5, 0.3),
                                   (0, 0.5, 0.9), (1, 0.5, 0.0), (0, 0.0, 0.0)])
def test_fp32_coarse_cut_in_a_crowded_bucket(k, p, m):
    """fp32 top-p (and top-k with it): the coarse pass sums masses per eighth
    of a binade; the cut inside the bucket comes from the listed candidates.
    About three quarters of the mass sits in 5000 distinct values of one
    bucket, so p = 0.1 and 0.5 cut inside it and 0.9 below it; k inside it
    with p below, k below with p inside, both inside, min-p on top, and ties
    at the cut (300 copies of one value).  With a mask and without."""
    rng = np.random.default_rng(211)
    R, cols = 5, 40000
    x = crowded_fp32_rows(rng, R, cols, 5000)
    x[4, rng.choice(cols, 300, replace=False)] = np.float32(1.0) + np.float32(3000 * 2.0 ** -21)
    bits = x.view(np.uint32)
    mask = workloads.pack_allowed(rng.random((R, cols)) < 0.9, (cols + 31) // 32, rng)
    say(f"[gpu] fp32 coarse cut k={k} p={p} m={m}")
    check_rows(bits, "float32", mask, None, 1.0, k, p, m, seed=7, offset=int(1000 * p) + k, min_exact=0.9)
    check_rows(bits, "float32", None, None, 0.9, k, p, m, seed=8, offset=int(1000 * p) + k, min_exact=0.9)


def test_fp32_coarse_bucket_edges_and_overflow():
    """Cuts on the edges of coarse buckets (values 1, 1.125 and 1.25 and the
    floats next to them, each repeated), and a bucket holding 20000 distinct
    values with the top-p cut inside it: more than the list holds, so the row
    takes the radix search."""
    rng = np.random.default_rng(212)
    cols = 30000
    x = rng.standard_normal((2, cols)).astype(np.float32) - np.float32(3.0)
    edges = np.array([1.0, 1.125, 1.25], np.float32)
    near = np.concatenate([edges, np.nextafter(edges, np.float32(0)), np.nextafter(edges, np.float32(9))])
    x[0, rng.choice(cols, near.size * 400, replace=False)] = np.repeat(near, 400)
    x[1, :] = np.float32(-4.0)
    x[1, rng.choice(cols, 20000, replace=False)] = np.float32(1.0) + np.arange(20000, dtype=np.float32) * np.float32(2.0 ** -21)
    bits = x.view(np.uint32)
    for (k, p, seed) in ((0, 0.5, 1), (0, 0.2, 2), (0, 0.8, 3), (1000, 1.0, 4), (2400, 1.0, 5), (500, 0.7, 6)):
        say(f"[gpu] fp32 bucket edges / list overflow k={k} p={p}")
        check_rows(bits, "float32", None, None, 1.0, k, p, 0.0, seed=seed, offset=seed, min_exact=0.9)


def test_fp32_coarse_bucket_crowding_one_wave():
    """The draw lists the cut bucket's candidates per wave (wave w of the
    1024-thread block reads the groups g with g % 1024 in [64 w, 64 w + 64)).
    1500 distinct values of one bucket placed in wave 0's groups fill its
    region though the whole list would hold them: the row takes the radix
    search.  A second row spreads the same values over the row."""
    rng = np.random.default_rng(213)
    cols = 40000
    x = rng.standard_normal((2, cols)).astype(np.float32) - np.float32(3.0)
    g = np.arange(cols // 8)
    wave0 = np.flatnonzero((g % 1024) < 64)
    pos0 = (wave0[:, None] * 8 + np.arange(8)).reshape(-1)
    vals = np.float32(1.0) + np.arange(1500, dtype=np.float32) * np.float32(2.0 ** -21)
    x[0, rng.choice(pos0, 1500, replace=False)] = vals
    x[1, rng.choice(cols, 1500, replace=False)] = vals
    bits = x.view(np.uint32)
    for (k, p, seed) in ((0, 0.5, 1), (700, 1.0, 2), (300, 0.6, 3)):
        say(f"[gpu] fp32 list crowding one wave k={k} p={p}")
        check_rows(bits, "float32", None, None, 1.0, k, p, 0.0, seed=seed, offset=seed, min_exact=0.9)


@pytest.mark.parametrize("dtype", ["float16", "bfloat16"])
def test_short_rows_with_filters(dtype):
    """16-bit rows shorter than one 8-token group, or with a ragged last
    group, under top-k, top-p and min-p: the histogram pass reads such tokens
    one at a time."""
    rng = np.random.default_rng(23)
    for V in (1, 3, 7, 9, 15, 17):
        R = 24
        bits = random_logits(rng, dtype, R, V)
        allowed = rng.random((R, V)) < 0.7
        allowed[0] = False
        mask = workloads.pack_allowed(allowed, (V + 31) // 32, rng)
        say(f"[gpu] sampler short rows V={V} {dtype}")
        for (T, k, p, m, seed) in ((1.0, 2, 1.0, 0.0, 1), (0.8, 0, 0.5, 0.0, 2), (1.0, 3, 0.9, 0.1, 3)):
            tok = check_rows(bits, dtype, mask, None, T, k, p, m, seed=seed, offset=V, min_exact=0.9)
            assert tok[0] == -1


@pytest.mark.parametrize("dtype", ["float16", "bfloat16"])
def test_fuzz_filtered_16bit(dtype):
    """Seeded random shapes, masks, value spreads (including heavy ties) and
    filter settings on 16-bit rows: the histogram search and both draw forms
    (walk and list) against the oracle."""
    rng = np.random.default_rng(29 if dtype == "float16" else 31)
    for case in range(12):
        R = int(rng.integers(1, 40))
        cols = int(rng.integers(1, 6000))
        ties = bool(rng.integers(0, 2))
        bits = random_logits(rng, dtype, R, cols, sigma=float(rng.choice([0.3, 2.0, 8.0])), ties=ties)
        density = rng.uniform(0.0, 1.0, (R, 1))
        mask = workloads.pack_allowed(rng.random((R, cols)) < density, (cols + 31) // 32 + int(rng.integers(0, 2)), rng)
        V = int(rng.integers(1, cols + 1))
        T = rng.choice([0.5, 1.0, 1.7], R).astype(np.float32)
        k = rng.choice([0, 1, 5, 50, 400, 10000], R).astype(np.int32)
        p = rng.choice([1.0, 0.99, 0.9, 0.5, 0.1], R).astype(np.float32)
        m = rng.choice([0.0, 0.0, 0.05], R).astype(np.float32)
        say(f"[gpu] sampler fuzz {dtype} case {case}: R={R} cols={cols} V={V} ties={ties}")
        check_rows(bits, dtype, mask, V, T, k, p, m, seed=100 + case, offset=case, min_exact=0.9)


@pytest.mark.parametrize("dtype", ["float16", "bfloat16"])
def test_kept_tokens_crowding_one_wave(dtype):
    """The listed draw gives each wave of the block a region of 2048 entries.
    Here every kept token lies in groups that one wave reads (thread t reads
    groups t, t + 1024, ...; wave 0 those with t < 64), 8000 of them, so that
    wave's region overflows and the row must take the walk instead."""
    rng = np.random.default_rng(37)
    R, cols = 4, 128000
    x = rng.standard_normal((R, cols)).astype(np.float32) - np.float32(12.0)
    group = np.arange(cols) // 8
    x[:, (group % 1024) < 64] += np.float32(16.0)      # wave 0's groups: 8000 tokens around +4
    if dtype == "float16":
        bits = x.astype(np.float16).view(np.uint16)
    else:
        b = x.view(np.uint32)
        bits = ((b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
    say(f"[gpu] sampler kept tokens crowding one wave {dtype}")
    check_rows(bits, dtype, None, None, 1.0, 0, 0.999, 0.0, seed=41, offset=0, min_exact=0.75, workspace=None)
    check_rows(bits, dtype, None, None, 1.0, 6000, 1.0, 0.0, seed=42, offset=1, min_exact=0.75, workspace=None)


@pytest.mark.parametrize("dtype", ["float32", "float16", "bfloat16"])
def test_segmented_rows_ties_and_sparse_candidates(dtype):
    """Few rows without filters are split into segments whose answers merge
    through one atomic maximum per row: equal maxima in several segments go
    to the lowest index, a row whose only candidates sit in one segment
    still finds them, and a row with none gets -1."""
    rng = np.random.default_rng(43)
    R, cols = 6, 70001
    x = rng.standard_normal((R, cols)).astype(np.float32)
    x[0, [100, 5000, 40000, 69999]] = 9.0          # equal maxima in four segments
    x[1, [69999, 3]] = 9.0
    allowed = np.ones((R, cols), bool)
    allowed[2] = False
    allowed[2, 50000:50010] = True                 # candidates in one segment only
    allowed[3] = False                             # none at all
    allowed[4, ::2] = False
    if dtype == "float32":
        bits = x.view(np.uint32)
    elif dtype == "float16":
        bits = x.astype(np.float16).view(np.uint16)
    else:
        b = x.view(np.uint32)
        bits = ((b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
    mask = workloads.pack_allowed(allowed, (cols + 31) // 32, rng)
    say(f"[gpu] sampler segmented rows {dtype}")
    # greedy through a per-row temperature array (all zero): a launch of scalar
    # greedy rows is split only at one or two rows, an array makes it split here
    tok = check_rows(bits, dtype, mask, None, np.zeros(R, np.float32), 0, 1.0, 0.0, seed=1, offset=0,
                     min_exact=1.0)
    assert tok[0] == 100 and tok[1] == 3 and 50000 <= tok[2] < 50010 and tok[3] == -1
    one = check_rows(bits[:1], dtype, mask[:1], None, 0.0, 0, 1.0, 0.0, seed=1, offset=0, min_exact=1.0)
    assert one[0] == 100
    tok = check_rows(bits, dtype, mask, None, 1.3, 0, 1.0, 0.0, seed=2, offset=5)
    assert tok[3] == -1 and 50000 <= tok[2] < 50010


def test_segmented_rows_in_a_graph():
    """The segmented launch (clear, sample, finish: three kernels, no memset)
    captured in a HIP graph replays to the eager tokens, several times, with
    other work between replays."""
    rng = np.random.default_rng(47)
    R, cols = 8, 40000
    bits = random_logits(rng, "bfloat16", R, cols)
    mask = workloads.pack_allowed(rng.random((R, cols)) < 0.4, (cols + 31) // 32, rng)
    dl = dev_logits(bits, "bfloat16")
    dm = torch.from_numpy(mask).to("cuda")
    temp = torch.from_numpy(rng.choice([0.0, 0.8, 1.2], R).astype(np.float32)).to("cuda")
    want = [mb.mi_apply_bitmask_sample(dl, dm, None, temperature=temp, seed=3, offset=k).cpu() for k in range(3)]
    say("[gpu] sampler segmented rows in a graph")
    outs = [torch.empty(R, dtype=torch.int64, device="cuda") for _ in range(3)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for k in range(3):
                mb.mi_apply_bitmask_sample(dl, dm, None, temperature=temp, seed=3, offset=k, out=outs[k])
    torch.cuda.synchronize()
    for rep in range(3):
        for o in outs:
            o.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        for k in range(3):
            assert torch.equal(outs[k].cpu(), want[k]), (rep, k)
        (dl.float() * 2).sum().item()
    del g
    check_rows(bits, "bfloat16", mask, None, temp.cpu().numpy(), 0, 1.0, 0.0, seed=3, offset=0)


def test_rows_split_over_launches():
    """More than 2^20 rows go out in several launches: the generator's row
    counter and the per-row parameter arrays continue across the split."""
    rng = np.random.default_rng(13)
    R, cols = (1 << 20) + 5, 8
    bits = random_logits(rng, "float32", R, cols)
    mask = rng.integers(1, 256, size=(R, 1)).astype(np.int32)
    T = rng.uniform(0.5, 1.5, R).astype(np.float32)
    k = rng.choice([0, 3], R).astype(np.int32)
    rows = [0, 1, (1 << 20) - 2, (1 << 20) - 1, 1 << 20, (1 << 20) + 1, R - 1]
    say(f"[gpu] sampler over {R} rows")
    check_rows(bits, "float32", mask, None, T, k, 1.0, 0.0, seed=17, offset=3, rows=rows, min_exact=1.0)


def test_long_rows():
    """Rows of 2^24 + 3 fp32 tokens (64 MB each): greedy on both and an
    unfiltered draw on one, against the oracle."""
    rng = np.random.default_rng(15)
    R, cols = 2, (1 << 24) + 3
    bits = random_logits(rng, "float32", R, cols)
    mask = workloads.pack_allowed(rng.random((R, cols)) < 0.5, (cols + 31) // 32, rng)
    say(f"[gpu] sampler on {R} rows of {cols} fp32 tokens")
    check_rows(bits, "float32", mask, None, 0.0, 0, 1.0, 0.0, seed=1, offset=0, min_exact=1.0)
    check_rows(bits, "float32", mask, None, 1.0, 0, 1.0, 0.0, seed=1, offset=1, rows=[1], min_exact=1.0)


@pytest.mark.parametrize("dtype", ["float32", "float16", "bfloat16"])
def test_non_finite_logits_are_not_candidates(dtype):
    """NaN (quiet and signalling patterns), +inf and -inf logits never count
    as candidates: rows with only NaNs take the first pass's fast form, rows
    with +inf its exact form; greedy and top-p agree with the oracle."""
    rng = np.random.default_rng(16)
    R, cols = 32, 1000
    bits = random_logits(rng, dtype, R, cols)
    if dtype == "float32":
        pos_inf, neg_inf, qnan, snan = 0x7F800000, 0xFF800000, 0x7FC00000, 0x7F800001
    elif dtype == "float16":
        pos_inf, neg_inf, qnan, snan = 0x7C00, 0xFC00, 0x7E00, 0x7C01
    else:
        pos_inf, neg_inf, qnan, snan = 0x7F80, 0xFF80, 0x7FC0, 0x7F81
    for r in range(R):
        idx = rng.choice(cols, 40, replace=False)
        kinds = [qnan, snan, neg_inf] + ([pos_inf] if r % 2 else [])   # odd rows also hold +inf
        for j, i in enumerate(idx):
            bits[r, i] = kinds[j % len(kinds)]
    bits[3, :] = snan                                                  # nothing finite at all
    mask = workloads.pack_allowed(rng.random((R, cols)) < 0.6, (cols + 31) // 32, rng)
    say(f"[gpu] sampler non-finite logits {dtype}")
    with np.errstate(invalid="ignore"):            # numpy notes the signalling NaNs it converts
        tok = check_rows(bits, dtype, mask, None, 0.0, 0, 1.0, 0.0, seed=3, offset=0, min_exact=1.0)
        assert tok[3] == -1
        check_rows(bits, dtype, mask, None, 1.0, 0, 0.8, 0.0, seed=3, offset=1)


def both_paths(dl, dm, vocab, **kw):
    """Tokens with one block per row and with the rows split through a workspace."""
    one = mb.mi_apply_bitmask_sample(dl, dm, vocab, workspace=None, **kw).cpu().numpy()
    split = mb.mi_apply_bitmask_sample(dl, dm, vocab, workspace="auto", **kw).cpu().numpy()
    return one, split


@pytest.mark.parametrize("dtype", ["float16", "bfloat16"])
def test_split_filtered_rows_equal_one_block_per_row(dtype):
    """A small batch of filtered 16-bit rows split over several blocks (the
    workspace) draws the same tokens as one block per row, bit for bit: the
    cut comes from the same counts and the draw from the same Gumbel keys.
    Batch sizes 1 to 32, ragged and masked rows, rows with no candidate,
    heavy ties, every filter alone and together, and per-row parameters that
    mix greedy, unfiltered and filtered rows in one batch."""
    rng = np.random.default_rng(67 if dtype == "float16" else 71)
    shapes = ((1, 128000, None), (3, 50257, None), (16, 32000, 31990), (32, 8192, None), (5, 70003, 70000))
    modes = (dict(top_k=50), dict(top_p=0.9), dict(min_p=0.05), dict(top_k=50, top_p=0.9, min_p=0.05),
             dict(top_k=1), dict(top_p=0.0), dict(top_k=1 << 20, top_p=0.999), dict(top_k=3000, temperature=0.5))
    for R, cols, V in shapes:
        ties = R in (3, 32)
        bits = random_logits(rng, dtype, R, cols, sigma=float(rng.choice([0.5, 2.0, 6.0])), ties=ties)
        allowed = rng.random((R, cols)) < rng.uniform(0.001, 0.9, (R, 1))
        if R > 2:
            allowed[1] = False
        mask = workloads.pack_allowed(allowed, (cols + 31) // 32, rng)
        dl = dev_logits(bits, dtype)
        dm = torch.from_numpy(mask).to("cuda")
        assert mb.sample_workspace_bytes(dl.dtype, R, V or cols) > 0
        for i, kw in enumerate(modes):
            say(f"[gpu] split vs one block {dtype} R={R} cols={cols} {kw}")
            one, split = both_paths(dl, dm, V, seed=5 + i, offset=R, **kw)
            assert np.array_equal(one, split), (R, cols, kw, np.flatnonzero(one != split)[:8])
            if R > 2:
                assert one[1] == -1
        T = torch.from_numpy(rng.choice([0.0, 0.7, 1.0, 1.3], R).astype(np.float32))
        k = torch.from_numpy(rng.choice([0, 1, 50, 5000], R).astype(np.int32))
        p = torch.from_numpy(rng.choice([1.0, 0.9, 0.5], R).astype(np.float32))
        m = torch.from_numpy(rng.choice([0.0, 0.0, 0.05], R).astype(np.float32))
        say(f"[gpu] split vs one block {dtype} R={R} cols={cols} per-row parameters")
        one, split = both_paths(dl, dm, V, temperature=T, top_k=k, top_p=p, min_p=m, seed=99, offset=7)
        assert np.array_equal(one, split), (R, cols, np.flatnonzero(one != split)[:8])


@pytest.mark.parametrize("dtype", ["float16", "bfloat16"])
def test_split_fuzz_equal_one_block(dtype):
    """Seeded random small batches (1 to 32 rows of 8192 to 200 000 tokens,
    ragged vocab, masks of random density, value spreads with and without
    heavy ties, per-row parameters mixing every mode): the split path and one
    block per row draw the same tokens."""
    rng = np.random.default_rng(97 if dtype == "float16" else 101)
    for case in range(8):
        R = int(rng.integers(1, 33))
        cols = int(rng.integers(8192, 200001))
        V = int(rng.integers(8192, cols + 1))
        ties = bool(rng.integers(0, 2))
        bits = random_logits(rng, dtype, R, cols, sigma=float(rng.choice([0.3, 2.0, 8.0])), ties=ties)
        allowed = rng.random((R, cols)) < rng.uniform(0.0, 1.0, (R, 1))
        mask = workloads.pack_allowed(allowed, (cols + 31) // 32 + int(rng.integers(0, 3)), rng)
        dl = dev_logits(bits, dtype)
        dm = torch.from_numpy(mask).to("cuda")
        T = torch.from_numpy(rng.choice([0.0, 0.5, 1.0, 1.7], R).astype(np.float32))
        k = torch.from_numpy(rng.choice([0, 1, 5, 50, 400, 100000], R).astype(np.int32))
        p = torch.from_numpy(rng.choice([1.0, 0.99, 0.9, 0.5, 0.1, 0.0], R).astype(np.float32))
        m = torch.from_numpy(rng.choice([0.0, 0.0, 0.05, 0.5], R).astype(np.float32))
        say(f"[gpu] split fuzz {dtype} case {case}: R={R} cols={cols} V={V} ties={ties}")
        one, split = both_paths(dl, dm, V, temperature=T, top_k=k, top_p=p, min_p=m, seed=300 + case, offset=case)
        assert np.array_equal(one, split), (case, np.flatnonzero(one != split)[:8])


def test_split_parameter_edges_equal_one_block():
    """Parameter edges through the split path, against one block per row:
    an infinite temperature (every filter keeps all), NaN top-p and min-p
    (disabled), top-p <= 0 and min-p >= 1 (the largest value and its ties),
    a row with a single candidate and a row with none, per-row parameters
    in one batch of 8 bf16 rows of 20 000 tokens with heavy ties."""
    rng = np.random.default_rng(103)
    R, cols = 8, 20000
    bits = random_logits(rng, "bfloat16", R, cols, sigma=1.0, ties=True)
    allowed = rng.random((R, cols)) < 0.5
    allowed[6] = False
    allowed[6, 12345] = True          # one candidate
    allowed[7] = False                # none
    mask = workloads.pack_allowed(allowed, (cols + 31) // 32, rng)
    dl = dev_logits(bits, "bfloat16")
    dm = torch.from_numpy(mask).to("cuda")
    inf, nan = float("inf"), float("nan")
    T = torch.tensor([inf, 1.0, 1.0, 1.0, 0.7, 1.3, 1.0, 1.0], dtype=torch.float32)
    k = torch.tensor([10, 0, 0, 0, 3, 0, 5, 5], dtype=torch.int32)
    p = torch.tensor([0.5, nan, 0.0, -1.0, 1.0, 0.9, 0.9, 0.9], dtype=torch.float32)
    m = torch.tensor([0.1, nan, 0.0, 0.0, 1.0, 2.0, 0.0, 0.0], dtype=torch.float32)
    for seed in (1, 2, 3):
        say(f"[gpu] split parameter edges seed {seed}")
        one, split = both_paths(dl, dm, None, temperature=T, top_k=k, top_p=p, min_p=m, seed=seed, offset=seed)
        assert np.array_equal(one, split), (seed, one, split)
        assert split[6] == 12345 and split[7] == -1


@pytest.mark.parametrize("dtype", ["float16", "bfloat16"])
def test_split_filtered_rows_against_the_oracle(dtype):
    """The split path against the oracle itself: 4 rows of the B=256 bf16
    shape (or fp16 rows of 32000), with masks, under each filter."""
    rng = np.random.default_rng(73)
    R, cols = (4, 128256) if dtype == "bfloat16" else (8, 32000)
    bits = random_logits(rng, dtype, R, cols)
    allowed = rng.random((R, cols)) < rng.uniform(0.01, 0.6, (R, 1))
    mask = workloads.pack_allowed(allowed, (cols + 31) // 32 + 1, rng)
    V = cols - 256 if dtype == "bfloat16" else None
    for (T, k, p, m, seed) in ((1.0, 50, 1.0, 0.0, 1), (1.0, 0, 0.9, 0.0, 2), (0.8, 0, 1.0, 0.1, 3),
                               (1.2, 40, 0.95, 0.02, 4)):
        say(f"[gpu] split path vs oracle {dtype} T={T} k={k} p={p} m={m}")
        check_rows(bits, dtype, mask, V, T, k, p, m, seed=seed, offset=seed, min_exact=0.9)


@pytest.mark.parametrize("dtype", ["float16", "bfloat16"])
def test_split_filtered_long_rows(dtype):
    """Rows of 2^21 + 5 tokens: the histogram pass needs 33 segments of under
    65536 tokens each (more than its usual 8 per row), with a ragged last
    segment.  Split and one-block tokens agree bit for bit, and the split
    tokens pass the oracle."""
    rng = np.random.default_rng(89)
    R, cols = 2, (1 << 21) + 5
    bits = random_logits(rng, dtype, R, cols)
    mask = workloads.pack_allowed(rng.random((R, cols)) < 0.4, (cols + 31) // 32, rng)
    dl = dev_logits(bits, dtype)
    dm = torch.from_numpy(mask).to("cuda")
    for i, kw in enumerate((dict(top_k=40), dict(top_p=0.8), dict(top_k=500, top_p=0.95, min_p=0.01))):
        say(f"[gpu] split long rows {dtype} {kw}")
        one, split = both_paths(dl, dm, None, seed=21 + i, offset=i, **kw)
        assert np.array_equal(one, split), (kw, one, split)
    check_rows(bits, dtype, mask, None, 1.0, 40, 0.8, 0.0, seed=30, offset=0, min_exact=1.0)


def test_split_workspace_reused_and_dirty():
    """An explicit workspace, filled with garbage first, serves two calls in a
    row, the second with fewer rows: its contents on entry do not matter."""
    rng = np.random.default_rng(79)
    bits = random_logits(rng, "bfloat16", 16, 40000)
    dl = dev_logits(bits, "bfloat16")
    ws = torch.full((mb.sample_workspace_bytes(torch.bfloat16, 16, 40000),), 0xFF, dtype=torch.uint8, device="cuda")
    for R in (16, 5):
        say(f"[gpu] split workspace reused, {R} rows")
        want = mb.mi_apply_bitmask_sample(dl[:R], None, None, top_k=20, top_p=0.8, seed=3, workspace=None)
        got = mb.mi_apply_bitmask_sample(dl[:R], None, None, top_k=20, top_p=0.8, seed=3, workspace=ws)
        assert torch.equal(want, got)


def test_split_filtered_rows_in_a_graph():
    """The split path's five kernels captured in a HIP graph (workspace
    allocated during capture) replay to the eager tokens three times, with
    unrelated eager work in between."""
    rng = np.random.default_rng(83)
    bits = random_logits(rng, "float16", 8, 32000)
    dl = dev_logits(bits, "float16")
    modes = (dict(top_k=50), dict(top_p=0.9, min_p=0.05))
    want = [mb.mi_apply_bitmask_sample(dl, None, None, seed=11, **kw).cpu() for kw in modes]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        outs = [mb.mi_apply_bitmask_sample(dl, None, None, seed=11, **kw) for kw in modes]   # warm-up
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = [mb.mi_apply_bitmask_sample(dl, None, None, seed=11, **kw) for kw in modes]
    for rep in range(3):
        say(f"[gpu] split path graph replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        for k in range(len(modes)):
            assert torch.equal(outs[k].cpu(), want[k]), (rep, modes[k])
        (dl.float() * 2).sum().item()
    del g


@pytest.mark.parametrize("T", [1.0, 0.11, 0.1, 0.02])
def test_fp32_fused_maximum_rescale_and_fallback(T):
    """fp32 rows of 1024-thread blocks take the row maximum from the coarse
    pass itself: each bucket's masses are summed relative to the bucket's
    largest value and rescaled to the maximum after the pass.  Row 0 holds
    its maximum 8.0 at the bottom of the bucket [8, 9): at T = 0.11 the top
    bucket's rescale is 2^13.1, at T = 0.1 it is 2^14.4, past the 2^14 at
    which the pass runs again relative to the maximum.  Row 1 has logits
    around 600 (buckets 64 wide: the pass runs again at every temperature
    here), row 2 negative logits with the maximum at a bucket's top edge,
    row 3 the maximum 500 times, row 4 a wide spread, row 5 no candidate.
    Against the oracle."""
    rng = np.random.default_rng(217)
    R, cols = 6, 20000
    x = rng.standard_normal((R, cols)).astype(np.float32)
    x[0] = rng.uniform(5.0, 7.99, cols).astype(np.float32)
    x[0, rng.choice(cols, 3, replace=False)] = np.float32(8.0)
    x[1] = np.float32(600.0) + rng.standard_normal(cols).astype(np.float32) * np.float32(3.0)
    x[2] = -np.abs(x[2]) - np.float32(1.0)
    x[2, 17] = np.float32(-1.0)
    x[3, rng.choice(cols, 500, replace=False)] = np.float32(4.5)
    x[4] *= np.float32(4.0)
    bits = x.view(np.uint32)
    allowed = rng.random((R, cols)) < 0.95
    allowed[:5, 0] = True
    allowed[0, x[0] == 8.0] = True
    allowed[5] = False
    mask = workloads.pack_allowed(allowed, (cols + 31) // 32, rng)
    for i, (k, p, m) in enumerate(((0, 0.9, 0.0), (0, 0.5, 0.0), (50, 0.9, 0.0), (0, 0.9, 0.05), (20, 1.0, 0.1))):
        say(f"[gpu] fp32 fused maximum T={T} k={k} p={p} m={m}")
        tok = check_rows(bits, "float32", mask, None, T, k, p, m, seed=31 + i, offset=i, min_exact=0.8)
        assert tok[5] == -1


def test_fp32_rows_past_the_fused_maximum_limit():
    """fp32 rows longer than 2^18 tokens (the most whose fixed-point bucket
    masses relative to the bucket's top fit 64 bits) take the maximum in a
    pass of its own before the coarse pass.  Against the oracle."""
    rng = np.random.default_rng(219)
    R, cols = 2, 300001
    x = rng.standard_normal((R, cols)).astype(np.float32) * np.float32(2.0)
    bits = x.view(np.uint32)
    for i, (k, p, m) in enumerate(((0, 0.9, 0.0), (50, 0.9, 0.02))):
        say(f"[gpu] fp32 rows of {cols} tokens k={k} p={p} m={m}")
        check_rows(bits, "float32", None, None, 1.0, k, p, m, seed=41 + i, offset=i, min_exact=0.5)


@pytest.mark.parametrize("dtype", ["float32", "float16", "bfloat16"])
def test_greedy_many_rows(dtype):
    """Greedy batches of more than 256 rows run the max-pass kernel in
    128-thread blocks: 300 ragged rows of 3001 tokens with ties, masks, a row
    without candidates, and NaN and infinite logits among the allowed
    tokens (never candidates).  Exact against the oracle's argmax (lowest
    index among ties)."""
    rng = np.random.default_rng(223)
    R, cols = 300, 3001
    bits = random_logits(rng, dtype, R, cols, ties=True)
    pos_inf, qnan = {"float32": (0x7F800000, 0x7FC00000), "float16": (0x7C00, 0x7E00),
                     "bfloat16": (0x7F80, 0x7FC0)}[dtype]
    for r in range(0, R, 7):
        bits[r, rng.choice(cols, 5, replace=False)] = [qnan, pos_inf, qnan, pos_inf, qnan]
    allowed = rng.random((R, cols)) < 0.3
    allowed[11] = False                                  # no candidate: -1
    mask = workloads.pack_allowed(allowed, (cols + 31) // 32, rng)
    say(f"[gpu] greedy, {R} rows {dtype}")
    with np.errstate(invalid="ignore"):
        tok = check_rows(bits, dtype, mask, None, 0.0, 0, 1.0, 0.0, seed=1, offset=0, min_exact=1.0)
        assert tok[11] == -1
        check_rows(bits, dtype, None, 2990, -2.0, 0, 1.0, 0.0, seed=1, offset=0, min_exact=1.0)


def mixed_density_mask(rng, R, cols, V, pad_words=0):
    """Masks of R rows mixing the kinds a grammar batch holds: dense rows
    (30 % to all of the tokens allowed), sparse rows (a few hundred to 4096
    allowed), rows allowing exactly 4096 and 4097 tokens below V (either
    side of the sparse-row limit) and rows allowing none; pad_words more
    words per row than the columns need, holding random bits."""
    allowed = np.zeros((R, cols), dtype=bool)
    kind = rng.choice(4, R, p=[0.25, 0.65, 0.05, 0.05])
    for r in range(R):
        if kind[r] == 0:
            allowed[r] = rng.random(cols) < rng.uniform(0.3, 1.0)
        elif kind[r] == 1:
            allowed[r, rng.choice(V, int(rng.integers(200, 4097)), replace=False)] = True
        elif kind[r] == 2:
            allowed[r, rng.choice(V, 4096 + (r & 1), replace=False)] = True
    return workloads.pack_allowed(allowed, (cols + 31) // 32 + pad_words, rng)


@pytest.mark.parametrize("dtype", ["float16", "bfloat16"])
def test_heavy_rows_first_tokens_do_not_depend_on_the_order(dtype):
    """Filtered batches of 257 to 8192 rows of more than 16 384 tokens
    (512-thread blocks up to 65 536 tokens, 1024-thread blocks beyond),
    given a workspace, hand out their dense rows first (a pass marks each
    row dense or sparse from its mask; every wave then finds its block's row
    by rank), so a row's block depends on the whole batch.  Its token must
    not: the batch without a workspace (row order), and a prefix of it
    (ordered differently, or not at all at 256 rows and fewer), draw the
    same tokens, for every mode that orders (top-p, min-p, the filters
    together, per-row parameters) and top-k alone, which does not; ragged
    vocab, padded mask rows, rows either side of the sparse-row limit and
    rows allowing nothing."""
    rng = np.random.default_rng(227 if dtype == "float16" else 229)
    modes = (dict(top_p=0.9), dict(min_p=0.05, top_p=0.95), dict(top_k=50, top_p=0.9, min_p=0.05), dict(top_k=50),
             dict(top_p=0.5, temperature=0.7))
    for R, cols, V, prefixes in ((1024, 32000, None, (1000, 600, 256)), (600, 50257, 50000, (257, 200)),
                                 (2048, 20000, 19999, (1500, 256)), (300, 70001, 70000, (257, 256))):
        bits = random_logits(rng, dtype, R, cols, sigma=float(rng.choice([1.0, 3.0])), ties=R == 600)
        mask = mixed_density_mask(rng, R, cols, V or cols, pad_words=3 if R == 2048 else 0)
        dl = dev_logits(bits, dtype)
        dm = torch.from_numpy(mask).to("cuda")
        T = torch.from_numpy(rng.choice([0.0, 0.8, 1.0, 1.5], R).astype(np.float32)).to("cuda")
        k = torch.from_numpy(rng.choice([0, 1, 40, 3000], R).astype(np.int32)).to("cuda")
        p = torch.from_numpy(rng.choice([1.0, 0.95, 0.6], R).astype(np.float32)).to("cuda")
        m = torch.from_numpy(rng.choice([0.0, 0.0, 0.1], R).astype(np.float32)).to("cuda")
        assert mb.sample_workspace_bytes(TORCH[dtype][1], R, V or cols) > 0
        for i, kw in enumerate(modes + ("per-row",)):
            say(f"[gpu] heavy rows first {dtype} R={R} cols={cols} V={V} {kw}")
            if kw == "per-row":
                call = lambda n, ws="auto": mb.mi_apply_bitmask_sample(
                    dl[:n], dm[:n], V, temperature=T[:n], top_k=k[:n], top_p=p[:n], min_p=m[:n], seed=5, offset=1,
                    workspace=ws).cpu().numpy()
            else:
                call = lambda n, ws="auto", kw=kw, i=i: mb.mi_apply_bitmask_sample(
                    dl[:n], dm[:n], V, seed=17 + i, offset=R, workspace=ws, **kw).cpu().numpy()
            whole = call(R)
            natural = call(R, None)
            assert np.array_equal(whole, natural), (R, kw, np.flatnonzero(whole != natural)[:8])
            for n in prefixes:
                part = call(n)
                assert np.array_equal(whole[:n], part), (R, n, kw, np.flatnonzero(whole[:n] != part)[:8])
        del dl, dm


def test_heavy_rows_first_largest_batch():
    """8192 rows (the most that are ordered) against 8193 (taken in row
    order): the first 8192 tokens agree, with top-p and min-p."""
    rng = np.random.default_rng(231)
    R, cols = 8193, 16400
    bits = random_logits(rng, "bfloat16", R, cols)
    mask = mixed_density_mask(rng, R, cols, cols)
    dl = dev_logits(bits, "bfloat16")
    dm = torch.from_numpy(mask).to("cuda")
    assert mb.sample_workspace_bytes(torch.bfloat16, R, cols) == 0
    assert mb.sample_workspace_bytes(torch.bfloat16, 8192, cols) > 0
    say("[gpu] heavy rows first: 8193 rows against their first 8192")
    whole = mb.mi_apply_bitmask_sample(dl, dm, None, top_p=0.9, min_p=0.02, seed=9).cpu().numpy()
    part = mb.mi_apply_bitmask_sample(dl[:8192], dm[:8192], None, top_p=0.9, min_p=0.02, seed=9).cpu().numpy()
    assert np.array_equal(whole[:8192], part), np.flatnonzero(whole[:8192] != part)[:8]


def test_heavy_rows_first_against_the_oracle():
    """The ordered path against the oracle directly: 300 fp16 rows of 17 000
    tokens of mixed density, top-p with min-p, and per-row parameters; 260
    bf16 rows of 66 000 tokens (1024-thread blocks), top-k alone."""
    rng = np.random.default_rng(233)
    R, cols = 300, 17000
    bits = random_logits(rng, "float16", R, cols)
    mask = mixed_density_mask(rng, R, cols, cols)
    say("[gpu] heavy rows first against the oracle, top-p 0.9 min-p 0.05")
    check_rows(bits, "float16", mask, None, 1.0, 0, 0.9, 0.05, seed=3, offset=4)
    lb = random_logits(rng, "bfloat16", 260, 66000)
    lm = mixed_density_mask(rng, 260, 66000, 66000)
    assert mb.sample_workspace_bytes(torch.bfloat16, 260, 66000) > 0
    say("[gpu] heavy rows first against the oracle, 260 bf16 rows of 66000, top-k 40")
    check_rows(lb, "bfloat16", lm, None, 1.0, 40, 1.0, 0.0, seed=6, offset=2)
    T = rng.choice([0.0, 0.7, 1.3], R).astype(np.float32)
    p = rng.choice([1.0, 0.8, 0.3], R).astype(np.float32)
    say("[gpu] heavy rows first against the oracle, per-row parameters")
    check_rows(bits, "float16", mask, None, T, 0, p, 0.0, seed=4, offset=5)


def test_heavy_rows_first_dirty_workspace_and_graph():
    """The ordering workspace, filled with garbage, serves two calls in a row
    (the second with fewer rows); then the two kernels of the ordered path,
    captured in a HIP graph with the workspace allocated during capture,
    replay to the tokens of row order three times, with eager work in
    between."""
    rng = np.random.default_rng(239)
    R, cols = 1024, 32000
    bits = random_logits(rng, "bfloat16", R, cols)
    dl = dev_logits(bits, "bfloat16")
    dm = torch.from_numpy(mixed_density_mask(rng, R, cols, cols)).to("cuda")
    ws = torch.full((mb.sample_workspace_bytes(torch.bfloat16, R, cols),), 0xFF, dtype=torch.uint8, device="cuda")
    for n in (R, 300):
        say(f"[gpu] ordering workspace reused, {n} rows")
        want = mb.mi_apply_bitmask_sample(dl[:n], dm[:n], None, top_p=0.9, seed=3, workspace=None)
        got = mb.mi_apply_bitmask_sample(dl[:n], dm[:n], None, top_p=0.9, seed=3, workspace=ws)
        assert torch.equal(want, got)
    modes = (dict(top_p=0.9), dict(top_k=50, top_p=0.9, min_p=0.05))
    want = [mb.mi_apply_bitmask_sample(dl, dm, None, seed=11, workspace=None, **kw).cpu() for kw in modes]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        outs = [mb.mi_apply_bitmask_sample(dl, dm, None, seed=11, **kw) for kw in modes]   # warm-up
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = [mb.mi_apply_bitmask_sample(dl, dm, None, seed=11, **kw) for kw in modes]
    for rep in range(3):
        say(f"[gpu] ordered path graph replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        for k in range(len(modes)):
            assert torch.equal(outs[k].cpu(), want[k]), (rep, modes[k])
        (dl.float() * 2).sum().item()
    del g
