"""The measurement script's contract, on the host (no GPU).

bench.py is what the headline figure comes from: these tests pin its
one-GPU refusal, its count of algorithmic bytes and its CPU baseline, and
that the committed HBM-counter summary it reads is well formed.
"""

import math
import pathlib
import subprocess
import sys

import numpy as np
import pytest

ROOT = pathlib.Path(__file__).resolve().parents[1]
sys.path.insert(0, str(ROOT))

import bench  # noqa: E402
import workloads  # noqa: E402


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                         timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout == ""


@pytest.mark.parametrize("rows,vocab,esize,out", [(128, 128000, 2, False), (1024, 32000, 2, True),
                                                   (2048, 262100, 4, False), (8, 50257, 2, False),
                                                   (1, 32000, 4, False)])
def test_effective_bytes(rows, vocab, esize, out):
    # mask words of the processed rows + one write pass (+ one read pass out of place)
    want = rows * math.ceil(vocab / 32) * 4 + rows * vocab * esize * (2 if out else 1)
    assert bench.effective_bytes(rows, vocab, esize, out) == want


def test_headline_effective_bytes_is_the_workloads():
    wl = workloads.mixed_bf16()
    assert len(wl.indices) == 128 and wl.vocab_size == 128000
    assert bench.effective_bytes(len(wl.indices), wl.vocab_size, 2) == 34_816_000


def test_counter_summary_is_well_formed():
    text = bench.PMC_SUMMARY.read_text()
    assert "traffic_bytes_per_dispatch:" in text and "kernel_source_sha256_16:" in text
    t = bench.counted_traffic()
    assert t is None or t > 34_816_000       # never below the algorithmic bytes


def test_cpu_baseline_runs_the_oracle():
    wl = workloads.mixed_bf16()
    eff = bench.effective_bytes(len(wl.indices), wl.vocab_size, 2)
    r = bench.cpu_baseline(wl, eff, 0.2)
    assert r["kind"] == "oracle" and r["cores"] == 1 and r["unit"] == "GB/s" and r["value"] > 0


def test_cold_rotation_counts_touched_bytes():
    # a launch of the headline touches its 128 indexed rows and their mask
    # words only: the rotation must cycle more than twice the Infinity Cache
    # in those bytes, not in the bytes each buffer set holds
    eff = bench.effective_bytes(128, 128000, 2)
    n = bench.cold_sets(eff)
    assert n * eff > 2 * bench.INFINITY_CACHE and (n - 1) * eff <= 2 * bench.INFINITY_CACHE
    assert bench.cold_sets(10 ** 12) == 2 and bench.cold_sets(1000, cap=64) == 64


def test_touched_lines_of_a_sparse_mask():
    # one allowed token per row in the first 128-byte line, one in the last:
    # two lines of logits per row plus the whole mask
    rows, V = 4, 1000
    bits = np.zeros((rows, V), dtype=bool)
    bits[:, 3] = True
    bits[:, V - 1] = True
    wl = workloads.Workload(name="t", dtype="bfloat16", logits=np.zeros((rows, V), np.uint16),
                            mask=workloads.pack_allowed(bits, (V + 31) // 32, np.random.default_rng(0)),
                            vocab_size=V, indices=None, fill_value=-math.inf, op="inplace")
    assert bench.touched_lines(wl, 2) == wl.mask.nbytes + rows * 2 * 128
