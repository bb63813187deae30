"""GPU parity: the HIP path against the CPU oracle, bit for bit.

Every case places the logits (and the out-of-place output) inside a larger
device buffer: random guard elements before and after, and random padding
columns between rows when the row pitch exceeds the width.  After the call
the WHOLE buffer is copied back and compared, with tolerance 0, against the
oracle applied to the same host buffer -- so a store outside the window, into
the padding, into a non-indexed row or past the vocab size fails the test
just like a wrong value inside it.

Named workloads run at their full sizes; the seeded fuzz draws small ragged
shapes (misaligned row pitches and base offsets, vocab tails, every index
form) for every kernel variant.
"""

import math
import sys

import numpy as np
import pytest

import oracle
import workloads
import packed_logit_bitmask_amd as mb

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TORCH_DTYPE = {"float32": torch.float32, "float16": torch.float16, "bfloat16": torch.bfloat16}
INT_VIEW = {"float32": (torch.int32, np.int32, np.uint32), "float16": (torch.int16, np.int16, np.uint16),
            "bfloat16": (torch.int16, np.int16, np.uint16)}
INPLACE_VARIANTS = ["auto", "scalar", "vec", "wronly", "vec_resident"]
OUT_VARIANTS = ["auto", "scalar", "vec"]


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu-marked tests need an MI355X")
    mb.load_library()
    return torch.device("cuda:0")


def to_device(bits: np.ndarray, dtype: str):
    tdt, ndt, _ = INT_VIEW[dtype]
    return torch.from_numpy(np.ascontiguousarray(bits).view(ndt)).to("cuda").view(TORCH_DTYPE[dtype])


def to_host(t, dtype: str) -> np.ndarray:
    tdt, _, udt = INT_VIEW[dtype]
    return t.view(tdt).cpu().numpy().view(udt)


class Placed:
    """A [rows, cols] window inside a flat buffer with guards and row padding."""

    def __init__(self, rng, bits: np.ndarray, dtype: str, stride: int, guard: int):
        rows, cols = bits.shape
        self.rows, self.cols, self.stride, self.guard, self.dtype = rows, cols, stride, guard, dtype
        udt = INT_VIEW[dtype][2]
        hi = 2**32 if udt == np.uint32 else 2**16
        n = 2 * guard + rows * stride + (0 if rows else 0)
        self.host = rng.integers(0, hi, size=max(n, 1), dtype=np.uint64).astype(udt)
        self.view(self.host)[:, :] = bits

    def view(self, flat):
        body = flat[self.guard:self.guard + self.rows * self.stride]
        return body.reshape(self.rows, self.stride)[:, :self.cols]

    def device(self):
        self.dev = to_device(self.host, self.dtype)
        return self.view(self.dev) if self.rows else self.dev[:0].view(0, self.cols)


def place_mask(rng, mask: np.ndarray, stride: int, guard: int):
    rows, mcols = mask.shape
    flat = rng.integers(0, 2**32, size=2 * guard + rows * stride + 1, dtype=np.uint64).astype(np.uint32)
    flat = flat.view(np.int32)
    body = flat[guard:guard + rows * stride].reshape(rows, stride)
    body[:, :mcols] = mask
    dev = torch.from_numpy(flat.copy()).to("cuda")
    dview = dev[guard:guard + rows * stride].view(rows, stride)[:, :mcols]
    return body[:, :mcols], dview


def run_inplace_case(rng, wl: workloads.Workload, variant: str, *, stride=None, guard=5, mask_pad=0,
                     indices_dev=None, expect_rows=None, stream=None):
    """Apply in place on the GPU and compare the whole buffer with the oracle."""
    stride = wl.cols if stride is None else stride
    P = Placed(rng, wl.logits, wl.dtype, stride, guard)
    hmask, dmask = place_mask(rng, wl.mask, wl.mask.shape[1] + mask_pad, 3)
    want = P.host.copy()
    idx = wl.indices if expect_rows is None else expect_rows
    oracle.apply_inplace(P.view(want), hmask, wl.dtype, wl.vocab_size,
                         None if idx is None else list(idx), wl.fill_value)
    dl = P.device()
    ind = indices_dev
    if ind is None and wl.indices is not None:
        ind = torch.from_numpy(np.asarray(wl.indices, dtype=np.int32)).to("cuda")
    mb.mi_apply_bitmask_inplace(dl, dmask, wl.vocab_size, ind, wl.fill_value, variant=variant, stream=stream)
    torch.cuda.synchronize()
    got = to_host(P.dev, wl.dtype)
    if not np.array_equal(got, want):
        bad = np.flatnonzero(got != want)
        raise AssertionError(f"{bad.size} elements differ; first at flat {bad[:8].tolist()}: "
                             f"got {got[bad[:4]].tolist()} want {want[bad[:4]].tolist()}")


def run_out_case(rng, wl: workloads.Workload, variant: str, *, stride=None, out_stride=None, guard=5,
                 out_guard=7, mask_pad=0, indices_dev=None, expect_rows=None):
    stride = wl.cols if stride is None else stride
    out_stride = wl.cols if out_stride is None else out_stride
    P = Placed(rng, wl.logits, wl.dtype, stride, guard)
    init = wl.out_init if wl.out_init is not None else np.zeros_like(wl.logits)
    O = Placed(rng, init, wl.dtype, out_stride, out_guard)
    hmask, dmask = place_mask(rng, wl.mask, wl.mask.shape[1] + mask_pad, 3)
    idx = wl.indices if expect_rows is None else expect_rows
    want = O.host.copy()
    O.view(want)[:, :] = oracle.apply_out(P.view(P.host), hmask, wl.dtype, wl.vocab_size,
                                          None if idx is None else list(idx), wl.fill_value)
    dl = P.device()
    do = O.device()
    ind = indices_dev
    if ind is None and wl.indices is not None:
        ind = torch.from_numpy(np.asarray(wl.indices, dtype=np.int32)).to("cuda")
    mb.mi_apply_bitmask_out(dl, dmask, do, wl.vocab_size, ind, wl.fill_value, variant=variant)
    torch.cuda.synchronize()
    got = to_host(O.dev, wl.dtype)
    src_after = to_host(P.dev, wl.dtype)
    assert np.array_equal(src_after, P.host), "out-of-place apply modified its input"
    if not np.array_equal(got, want):
        bad = np.flatnonzero(got != want)
        raise AssertionError(f"{bad.size} elements differ; first at flat {bad[:8].tolist()}")


# ----------------------------------------------------------------------------
# named workloads at full size
# ----------------------------------------------------------------------------

SMALL_NAMED = ["tiny", "tail_bf16", "mixed_bf16"]


@pytest.mark.parametrize("variant", INPLACE_VARIANTS)
@pytest.mark.parametrize("name", SMALL_NAMED)
def test_named_inplace(name, variant):
    say(f"[gpu] named {name} variant={variant}")
    wl = workloads.NAMED[name]()
    run_inplace_case(np.random.default_rng(1), wl, variant)


def test_mixed_bf16_sorted_indices_and_all_rows():
    rng = np.random.default_rng(2)
    say("[gpu] mixed_bf16 sorted indices / all rows")
    run_inplace_case(rng, workloads.mixed_bf16(sorted_indices=True), "auto")
    run_inplace_case(rng, workloads.mixed_bf16(n_indices=256), "auto")
    wl = workloads.mixed_bf16()
    wl.indices = None
    run_inplace_case(rng, wl, "auto")


@pytest.mark.parametrize("variant", OUT_VARIANTS)
def test_named_verify_fp16_out(variant):
    say(f"[gpu] named verify_fp16 out variant={variant}")
    run_out_case(np.random.default_rng(3), workloads.verify_fp16(), variant)


@pytest.fixture(scope="module")
def large():
    say("[gpu] drawing large_fp32 (2048 x 262144 fp32)")
    wl = workloads.large_fp32()
    want = wl.logits.copy()
    oracle.apply_inplace(want, wl.mask, wl.dtype, wl.vocab_size, None, wl.fill_value)
    dmask = torch.from_numpy(wl.mask).to("cuda")
    return wl, want, dmask


@pytest.mark.parametrize("variant", INPLACE_VARIANTS)
def test_named_large_fp32(large, variant):
    """The 2.2 GB workload, inside one device buffer with random guard words
    on both sides (4 KiB each): a store past either end of the tensor, as
    the widest vector instantiation could make, changes a guard."""
    wl, want, dmask = large
    say(f"[gpu] named large_fp32 variant={variant}")
    guard = 1024
    n = wl.rows * wl.cols
    g = np.random.default_rng(77).integers(0, 2**32, size=2 * guard, dtype=np.uint64).astype(np.uint32)
    buf = torch.empty(n + 2 * guard, dtype=torch.int32, device="cuda")
    buf[:guard] = torch.from_numpy(g[:guard].view(np.int32)).to("cuda")
    buf[guard + n:] = torch.from_numpy(g[guard:].view(np.int32)).to("cuda")
    buf[guard:guard + n] = torch.from_numpy(wl.logits.view(np.int32).reshape(-1)).to("cuda")
    d = buf[guard:guard + n].view(torch.float32).view(wl.rows, wl.cols)
    mb.mi_apply_bitmask_inplace(d, dmask, wl.vocab_size, None, wl.fill_value, variant=variant)
    torch.cuda.synchronize()
    assert np.array_equal(buf[:guard].cpu().numpy().view(np.uint32), g[:guard]), "store before the tensor"
    assert np.array_equal(buf[guard + n:].cpu().numpy().view(np.uint32), g[guard:]), "store past the tensor"
    got = to_host(d, wl.dtype)
    assert np.array_equal(got, want)
    del d, buf
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype,rows,cols,vocab", [
    ("bfloat16", 800, 40001, 39999),   # below 1 GB of writes: two vectors per lane, streaming stores
    ("float16", 700, 50003, None),
    ("float32", 500, 30001, 29990),
    ("float32", 4500, 60001, None),    # >= 1 GB of writes: four vectors per lane
])
def test_large_shapes_misaligned(dtype, rows, cols, vocab):
    rng = np.random.default_rng(rows)
    say(f"[gpu] large misaligned {dtype} [{rows},{cols}] vocab={vocab}")
    wl, _, _ = workloads.random_case(rng, dtype, rows, cols, vocab_size=vocab, density=0.3, specials=True)
    run_inplace_case(rng, wl, "auto", stride=cols + 3, guard=3)
    wl.indices = rng.permutation(rows)[: rows - 7].astype(np.int32)
    run_inplace_case(rng, wl, "vec", stride=cols + 1, guard=1)
    run_out_case(rng, wl, "auto", stride=cols + 2, out_stride=cols + 6, guard=2, out_guard=6)


# ----------------------------------------------------------------------------
# seeded fuzz: ragged shapes, every index form, every variant
# ----------------------------------------------------------------------------

def fuzz_case(seed):
    rng = np.random.default_rng(1000 + seed)
    dtype = ["float32", "float16", "bfloat16"][seed % 3]
    rows = int(rng.integers(1, 24))
    cols = int(rng.choice([1, 7, 31, 32, 33, 63, 64, 65, 100, 511, 1000, 2049, 4100, 9000]))
    cols = max(1, cols + int(rng.integers(-1, 2)))
    mask_cols = (cols + 31) // 32 + int(rng.integers(0, 3))
    mask_rows = rows + int(rng.integers(0, 3))
    limit = min(cols, 32 * mask_cols)
    vocab = [None, limit, int(rng.integers(0, limit + 1))][int(rng.integers(0, 3))]
    kind = ["none", "sorted", "unsorted", "empty", "dups"][int(rng.integers(0, 5))]
    n = {"none": None, "sorted": int(rng.integers(1, rows + 1)), "unsorted": int(rng.integers(1, rows + 1)),
         "empty": 0, "dups": int(rng.integers(1, rows + 1))}[kind]
    density = float(rng.choice([0.5, 0.02, 0.98, 0.0, 1.0]))
    wl, _, _ = workloads.random_case(rng, dtype, rows, cols, mask_rows=mask_rows, mask_cols=mask_cols,
                                     vocab_size=vocab, n_indices=n, density=density,
                                     fill_value=float(rng.choice([-math.inf, -1e4, 3.0, math.nan])))
    if kind == "sorted":
        wl.indices = np.sort(wl.indices)
    if kind == "dups":
        wl.indices = np.concatenate([wl.indices, wl.indices[:1]])
    stride = cols + int(rng.integers(0, 12))
    guard = int(rng.integers(0, 11))
    return rng, wl, stride, guard, kind


@pytest.mark.parametrize("seed", range(48))
def test_fuzz_inplace(seed):
    rng, wl, stride, guard, kind = fuzz_case(seed)
    for variant in INPLACE_VARIANTS:
        say(f"[gpu] fuzz inplace seed={seed} {wl.dtype} {wl.logits.shape} stride={stride} guard={guard} "
            f"vocab={wl.vocab_size} idx={kind} variant={variant}")
        run_inplace_case(rng, wl, variant, stride=stride, guard=guard, mask_pad=seed % 3)


@pytest.mark.parametrize("seed", range(36))
def test_fuzz_out(seed):
    rng, wl, stride, guard, kind = fuzz_case(seed)
    out_stride = wl.cols + int(rng.integers(0, 12))
    for variant in OUT_VARIANTS:
        say(f"[gpu] fuzz out seed={seed} {wl.dtype} {wl.logits.shape} stride={stride}/{out_stride} "
            f"vocab={wl.vocab_size} idx={kind} variant={variant}")
        run_out_case(rng, wl, variant, stride=stride, out_stride=out_stride, guard=guard,
                     out_guard=int(rng.integers(0, 9)), mask_pad=seed % 2)


# ----------------------------------------------------------------------------
# edge cases
# ----------------------------------------------------------------------------

def test_out_of_range_device_indices_are_skipped():
    rng = np.random.default_rng(7)
    wl, _, _ = workloads.random_case(rng, "bfloat16", 6, 300, mask_rows=5)
    dev_idx = torch.tensor([4, -1, 2, 5, 1 << 30, 0], dtype=torch.int32, device="cuda")
    say("[gpu] out-of-range device indices")
    for variant in INPLACE_VARIANTS:
        run_inplace_case(rng, wl, variant, indices_dev=dev_idx, expect_rows=[4, 2, 0])
    for variant in OUT_VARIANTS:
        run_out_case(rng, wl, variant, indices_dev=dev_idx, expect_rows=[4, 2, 0])


@pytest.mark.parametrize("n_list", [1, 1023, 1024, 1025, 3000])
def test_out_of_place_index_list_sizes(n_list):
    """Out of place with an index list: up to 1024 entries in one pass (each
    block looks for its row in the list), beyond that a copy then the in-place
    apply.  Lists on both sides of the limit, with duplicates, entries past
    the mask rows and past the logits rows, and negative entries; more logits
    rows than mask rows."""
    rng = np.random.default_rng(8000 + n_list)
    rows, mask_rows = 3100, 3050
    wl, _, _ = workloads.random_case(rng, "float16", rows, 700, mask_rows=mask_rows, vocab_size=690, density=0.3)
    valid = rng.permutation(mask_rows)[: max(1, n_list - 6)]
    extra = np.array([-1, mask_rows, rows - 1, rows, 1 << 30, int(valid[0])], dtype=np.int64)[: n_list - valid.size]
    idx = np.concatenate([valid, extra]).astype(np.int32)
    rng.shuffle(idx)
    expect = sorted({int(i) for i in idx if 0 <= i < mask_rows})
    say(f"[gpu] out of place, index list of {idx.size}")
    for variant in OUT_VARIANTS:
        run_out_case(rng, wl, variant, stride=703, out_stride=701, guard=2, out_guard=3,
                     indices_dev=torch.from_numpy(idx).to("cuda"), expect_rows=expect)


@pytest.mark.parametrize("dtype", ["float32", "bfloat16"])
def test_degenerate_shapes(dtype):
    rng = np.random.default_rng(8)
    say(f"[gpu] degenerate shapes {dtype}")
    for rows, cols, vocab in [(1, 1, None), (1, 1, 0), (3, 5, 0), (2, 32, 1), (1, 33, None), (5, 64, 63)]:
        wl, _, _ = workloads.random_case(rng, dtype, rows, cols, vocab_size=vocab)
        for variant in INPLACE_VARIANTS:
            run_inplace_case(rng, wl, variant, stride=cols + 1, guard=1)
        for variant in OUT_VARIANTS:
            run_out_case(rng, wl, variant, stride=cols + 2, out_stride=cols, guard=2)
    # zero rows
    wl, _, _ = workloads.random_case(rng, dtype, 0, 40, mask_rows=0)
    d = torch.empty(0, 40, dtype=TORCH_DTYPE[dtype], device="cuda")
    m = torch.empty(0, 2, dtype=torch.int32, device="cuda")
    mb.mi_apply_bitmask_inplace(d, m)
    mb.mi_apply_bitmask_out(d, m)
    torch.cuda.synchronize()


def test_all_ones_and_all_zero_masks():
    rng = np.random.default_rng(9)
    say("[gpu] all-ones / all-zero masks")
    for dens in (1.0, 0.0):
        for dtype in ("float32", "float16", "bfloat16"):
            wl, _, _ = workloads.random_case(rng, dtype, 4, 5000, density=dens, row_pad=0)
            for variant in INPLACE_VARIANTS:
                run_inplace_case(rng, wl, variant, stride=5003, guard=3)


def test_side_stream_and_graph_replay():
    rng = np.random.default_rng(10)
    wl = workloads.mixed_bf16(rows=16, vocab=4000, col_pad=24, word_pad=2)
    say("[gpu] side stream")
    s = torch.cuda.Stream()
    run_inplace_case(rng, wl, "auto", stream=s)
    say("[gpu] graph capture + replays")
    want = wl.logits.copy()
    oracle.apply_inplace(want, wl.mask, wl.dtype, wl.vocab_size, list(wl.indices), wl.fill_value)
    d = to_device(wl.logits, wl.dtype).view(wl.rows, wl.cols)
    pristine = d.clone()
    dm = torch.from_numpy(wl.mask).to("cuda")
    di = torch.from_numpy(wl.indices).to("cuda")
    g = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cs):
        mb.mi_apply_bitmask_inplace(d, dm, wl.vocab_size, di, wl.fill_value)  # warm-up outside capture
    torch.cuda.current_stream().wait_stream(cs)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        mb.mi_apply_bitmask_inplace(d, dm, wl.vocab_size, di, wl.fill_value)
    for rep in range(4):
        d.copy_(pristine)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_host(d, wl.dtype), want), f"replay {rep}"


def test_cross_phase_out_uses_any_alignment():
    # out and logits rows at different offsets modulo 16 bytes
    rng = np.random.default_rng(11)
    say("[gpu] out-of-place across alignment phases")
    for dtype in ("float32", "float16"):
        wl, _, _ = workloads.random_case(rng, dtype, 5, 777, vocab_size=700)
        for variant in OUT_VARIANTS:
            run_out_case(rng, wl, variant, stride=781, out_stride=779, guard=1, out_guard=6)


def test_xgrammar_surface_on_gpu():
    rng = np.random.default_rng(12)
    say("[gpu] XGrammar-compatible apply_token_bitmask_inplace on GPU tensors")
    for dtype in ("float32", "float16", "bfloat16"):
        wl, _, _ = workloads.random_case(rng, dtype, 6, 1000, mask_cols=34, n_indices=4)
        want = oracle.apply_inplace(np.array(wl.logits), wl.mask, dtype, 999, list(wl.indices))
        x = to_device(np.array(wl.logits), dtype).view(6, 1000)
        m = torch.from_numpy(np.ascontiguousarray(wl.mask)).to("cuda")
        mb.apply_token_bitmask_inplace(x, m, vocab_size=999, indices=list(wl.indices))
        torch.cuda.synchronize()
        assert np.array_equal(to_host(x, dtype), want)
    with pytest.raises(ValueError):
        mb.apply_token_bitmask_inplace(x, m.cpu())          # mixed devices: the caller copies the mask


# ----------------------------------------------------------------------------
# gated apply with the per-row report
# ----------------------------------------------------------------------------

def run_rows_case(rng, logits_bits, mask, dtype, vocab, gate, *, stride=None, shape3=None, report=True):
    rows, cols = logits_bits.shape
    stride = cols if stride is None else stride
    P = Placed(rng, logits_bits, dtype, stride, 4)
    hmask, dmask = place_mask(rng, mask, mask.shape[1] + 1, 2)
    want = P.host.copy()
    _, want_rep = oracle.apply_rows(P.view(want), hmask, dtype, vocab, gate, -math.inf)
    dl = P.device()
    if shape3 is not None:
        dl = P.dev[P.guard:P.guard + rows * stride].view(shape3[0], shape3[1], stride)[:, :, :cols]
    g = None if gate is None else torch.from_numpy(np.asarray(gate, dtype=np.int8)).to("cuda")
    rep = mb.mi_apply_bitmask_rows(dl, dmask, g, vocab, report=report)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(P.dev, dtype), want)
    if report:
        assert rep.cpu().numpy().tolist() == want_rep.tolist()


def test_rows_hand_cases_on_gpu():
    from _golden import build_case, load
    say("[gpu] gated apply: hand cases")
    for case in load()["rows_cases"]["cases"]:
        logits, mask = build_case(case)
        gate = None if case["gate"] is None else np.array(case["gate"], dtype=np.int8)
        run_rows_case(np.random.default_rng(0), logits, mask, case["dtype"], case["vocab_size"], gate)


def test_rows_verify_shape_with_gate_and_report():
    rng = np.random.default_rng(13)
    say("[gpu] gated apply: verify_fp16 shape as [256,4,32000] with random gate")
    wl = workloads.verify_fp16()
    gate = (rng.random(wl.rows) < 0.8).astype(np.int8)
    run_rows_case(rng, wl.logits, wl.mask, wl.dtype, None, gate, shape3=(256, 4))
    run_rows_case(rng, wl.logits, wl.mask, wl.dtype, None, None)
    run_rows_case(rng, wl.logits, wl.mask, wl.dtype, None, np.zeros(wl.rows, np.int8))
    run_rows_case(rng, wl.logits, wl.mask, wl.dtype, 0, gate)


@pytest.mark.parametrize("name", ["tail_bf16", "mixed_bf16", "tiny"])
def test_rows_named_with_garbage_tails(name):
    rng = np.random.default_rng(14)
    say(f"[gpu] gated apply: {name}")
    wl = workloads.NAMED[name]()
    gate = (rng.random(wl.rows) < 0.5).astype(np.int8)
    # zero the in-range bits of some rows so they are unsatisfiable; garbage past V stays
    V = oracle.resolve_vocab_size(wl.cols, wl.mask.shape[1], wl.vocab_size)
    mask = wl.mask.copy().view(np.uint32)
    W, t = (V + 31) // 32, V % 32
    for r in range(0, wl.rows, 3):
        mask[r, :W - (1 if t else 0)] = 0
        if t:
            mask[r, W - 1] &= np.uint32((0xFFFFFFFF << t) & 0xFFFFFFFF)
    run_rows_case(rng, wl.logits, mask.view(np.int32), wl.dtype, wl.vocab_size, gate, stride=wl.cols + 5)


@pytest.mark.parametrize("seed", range(12))
def test_rows_fuzz(seed):
    rng = np.random.default_rng(2000 + seed)
    dtype = ["float32", "float16", "bfloat16"][seed % 3]
    rows = int(rng.integers(1, 30))
    cols = int(rng.choice([5, 33, 100, 1000, 4097, 20000]))
    mask_cols = (cols + 31) // 32 + int(rng.integers(0, 2))
    wl, _, _ = workloads.random_case(rng, dtype, rows, cols, mask_cols=mask_cols,
                                     density=float(rng.choice([0.0, 0.001, 0.5])))
    vocab = [None, int(rng.integers(0, min(cols, 32 * mask_cols) + 1))][seed % 2]
    gate = None if seed % 4 == 0 else (rng.random(rows) < 0.6).astype(np.int8)
    say(f"[gpu] gated fuzz seed={seed} {dtype} [{rows},{cols}] vocab={vocab}")
    run_rows_case(rng, wl.logits, wl.mask, dtype, vocab, gate, stride=cols + int(rng.integers(0, 9)),
                  report=seed % 3 != 0)


# ----------------------------------------------------------------------------
# mask staging: host fill -> async upload on a side stream -> apply
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("depth", [1, 2, 3])
def test_staged_decode_loop(depth):
    say(f"[gpu] MaskStager depth={depth}")
    rng = np.random.default_rng(40 + depth)
    B, V, cols = 16, 5000, 5024
    stager = mb.MaskStager(B, V, depth=depth)
    compute = torch.cuda.Stream()
    w = torch.randn(256, cols, device="cuda", dtype=torch.float16)
    results = []
    with torch.cuda.stream(compute):
        for step in range(7):
            h = stager.host()
            bits = rng.random((B, V)) < rng.uniform(0.05, 0.9)
            mask_np = workloads.pack_allowed(bits, h.shape[1], rng)
            h.copy_(torch.from_numpy(mask_np))
            stager.upload()
            # the "forward": logits produced on the compute stream while the mask uploads
            a = torch.randn(B, 256, device="cuda", dtype=torch.float16)
            logits = a @ w
            keep_in = logits.clone()
            stager.apply_inplace(logits, vocab_size=V, stream=compute)
            results.append((keep_in, logits, mask_np))
    torch.cuda.synchronize()
    for step, (before, after, mask_np) in enumerate(results):
        src = before.view(torch.int16).cpu().numpy().view(np.uint16)
        want = oracle.apply_inplace(src.copy(), mask_np, "float16", V)
        assert np.array_equal(after.view(torch.int16).cpu().numpy().view(np.uint16), want), step


def test_grids_split_over_several_launches():
    """More row slots than one launch holds (2^24 - 1 blocks of one chunk):
    the host splits the grid, and every row is still applied exactly once.
    Also the gated apply with its report, whose extra block per row halves
    the slots a launch takes."""
    rng = np.random.default_rng(12)
    R, cols = (1 << 24) + 3, 8                   # 268 MB of bf16; one 16-byte vector per row
    bits = rng.integers(0, 1 << 16, size=(R, cols), dtype=np.uint16)
    mask = rng.integers(-(1 << 31), 1 << 31, size=(R, 1), dtype=np.int64).astype(np.int32)
    say(f"[gpu] {R} rows of 8 bf16 tokens, in place")
    x = to_device(bits, "bfloat16")
    m = torch.from_numpy(mask).to("cuda")
    mb.mi_apply_bitmask_inplace(x, m)
    want = oracle.apply_inplace(bits.copy(), mask, "bfloat16")
    got = to_host(x, "bfloat16")
    assert np.array_equal(got, want)
    del x, got, want

    R2 = (1 << 23) + 3
    b2 = bits[:R2].copy()
    gate = (rng.random(R2) < 0.7).astype(np.int8)
    gate[-1] = 1
    say(f"[gpu] {R2} rows, gated with the report")
    x = to_device(b2, "bfloat16")
    rep = mb.mi_apply_bitmask_rows(x, m[:R2], torch.from_numpy(gate).to("cuda"), report=True)
    want, want_any = oracle.apply_rows(b2.copy(), mask[:R2], "bfloat16", None, gate)
    assert np.array_equal(to_host(x, "bfloat16"), want)
    assert np.array_equal(rep.cpu().numpy(), want_any)


def test_longest_row():
    """One row at the column limit: 2^30 - 5 bf16 tokens (2 GB), a mask of
    2^25 words with garbage past V, applied in place (the buffer resources
    and chunk offsets of a single row at its largest)."""
    rng = np.random.default_rng(14)
    cols = (1 << 30) - 5
    bits = rng.integers(0, 1 << 16, size=(1, cols), dtype=np.uint16)
    mask = rng.integers(-(1 << 31), 1 << 31, size=(1, 1 << 25), dtype=np.int64).astype(np.int32)
    say(f"[gpu] one row of {cols} bf16 tokens")
    x = to_device(bits, "bfloat16")
    m = torch.from_numpy(mask).to("cuda")
    mb.mi_apply_bitmask_inplace(x, m)
    got = to_host(x, "bfloat16")
    del x
    oracle.apply_inplace(bits, mask, "bfloat16")
    assert np.array_equal(got, bits)


@pytest.mark.parametrize("dtype", ["float32", "float16", "bfloat16"])
def test_out_onto_its_own_input_is_the_inplace_apply(dtype):
    """out == logits with the same row pitch is the in-place apply (the
    out-of-place entry's documented alias rule): whole-buffer equality with
    the oracle's in-place result, with and without an index list, on an odd
    row pitch."""
    rng = np.random.default_rng(17)
    rows, cols = 40, 3001
    for n_idx in (None, 17):
        wl, _, _ = workloads.random_case(rng, dtype, rows, cols, vocab_size=2990, n_indices=n_idx, density=0.4,
                                         fill_value=-1e4)
        P = Placed(rng, wl.logits, wl.dtype, cols + 5, 3)
        hmask, dmask = place_mask(rng, wl.mask, wl.mask.shape[1], 3)
        want = P.host.copy()
        oracle.apply_inplace(P.view(want), hmask, wl.dtype, wl.vocab_size,
                             None if wl.indices is None else list(wl.indices), wl.fill_value)
        dl = P.device()
        ind = None if wl.indices is None else torch.from_numpy(np.asarray(wl.indices, np.int32)).to("cuda")
        say(f"[gpu] out onto its own input {dtype} indices={n_idx}")
        mb.mi_apply_bitmask_out(dl, dmask, dl, wl.vocab_size, ind, wl.fill_value)
        torch.cuda.synchronize()
        assert np.array_equal(to_host(P.dev, wl.dtype), want)
