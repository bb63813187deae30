"""The oracle's fill conversion against library conversions and the definition.

* binary32 / binary16: numpy's conversion of a float64 to float32 / float16
  rounds once, to nearest-even, with overflow to infinity -- the reading the
  oracle takes.  Checked on random doubles from every range that matters
  (normal, subnormal, underflow, overflow, exact ties).
* bfloat16: torch's float32 -> bfloat16 rounds to nearest-even; on doubles
  that are exact float32 values a single rounding from the double is the
  same, so the two must agree there.
* all three: every finite pattern of the format decodes to a double the
  oracle maps back to the same pattern, and the midpoint of two neighbours
  goes to the one with the even fraction (the definition of ties-to-even).
"""

import math

import numpy as np
import pytest
import torch

import oracle


def random_doubles(rng, n):
    parts = [
        rng.standard_normal(n) * 10.0 ** rng.integers(-45, 40, size=n),
        rng.uniform(-70000, 70000, n),
        rng.standard_normal(n) * 2.0 ** -24,
        rng.standard_normal(n) * 2.0 ** -140,
        rng.uniform(3.0e38, 3.5e38, n) * rng.choice([-1, 1], n),
    ]
    bits = rng.integers(0, 2**63, size=n, dtype=np.int64).view(np.float64)
    parts.append(bits[np.isfinite(bits)])
    return np.concatenate(parts)


@pytest.mark.parametrize("dtype,npt", [("float32", np.float32), ("float16", np.float16)])
def test_against_numpy_single_rounding(dtype, npt):
    rng = np.random.default_rng(11)
    xs = random_doubles(rng, 4000)
    width = np.uint32 if npt is np.float32 else np.uint16
    with np.errstate(over="ignore"):
        want = xs.astype(npt).view(width)
    for x, w in zip(xs.tolist(), want.tolist()):
        assert oracle.fill_bits(x, dtype) == w, (x, dtype)


def test_bfloat16_against_torch_on_exact_float32_values():
    rng = np.random.default_rng(12)
    f32 = np.concatenate([
        rng.integers(0, 2**32, size=20000, dtype=np.uint64).astype(np.uint32).view(np.float32),
        (rng.standard_normal(5000) * 100).astype(np.float32),
    ])
    f32 = f32[np.isfinite(f32)]
    want = torch.from_numpy(f32.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    for x, w in zip(f32.astype(np.float64).tolist(), want.tolist()):
        assert oracle.fill_bits(x, "bfloat16") == w, x


def decode_all(dtype):
    """Every finite non-negative pattern of a 16-bit format, decoded by numpy/torch."""
    pats = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    if dtype == "float16":
        vals = pats.view(np.float16).astype(np.float64)
    else:
        with np.errstate(invalid="ignore"):
            vals = (pats.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    keep = np.isfinite(vals) & (pats < 0x8000)
    return pats[keep].astype(np.int64), vals[keep]


@pytest.mark.parametrize("dtype", ["float16", "bfloat16"])
def test_round_trip_and_midpoints(dtype):
    pats, vals = decode_all(dtype)
    order = np.argsort(vals, kind="stable")
    pats, vals = pats[order], vals[order]
    for p, v in zip(pats.tolist(), vals.tolist()):
        assert oracle.fill_bits(v, dtype) == p
        assert oracle.fill_bits(-v, dtype) == p | 0x8000
    for (p0, v0), (p1, v1) in zip(zip(pats.tolist(), vals.tolist()), zip(pats[1:].tolist(), vals[1:].tolist())):
        mid = (v0 + v1) / 2.0          # exact in float64 for these formats
        even = p0 if p0 % 2 == 0 else p1
        assert oracle.fill_bits(mid, dtype) == even
        assert oracle.fill_bits(math.nextafter(mid, -math.inf), dtype) == p0
        assert oracle.fill_bits(math.nextafter(mid, math.inf), dtype) == p1


def test_float32_sampled_midpoints():
    rng = np.random.default_rng(13)
    pats = rng.integers(0, 0x7F7FFFFF, size=20000, dtype=np.int64)
    for p in pats.tolist():
        v0 = float(np.uint32(p).view(np.float32))
        v1 = float(np.uint32(p + 1).view(np.float32))
        assert oracle.fill_bits(v0, "float32") == p
        mid = (v0 + v1) / 2.0
        assert oracle.fill_bits(mid, "float32") == (p if p % 2 == 0 else p + 1)


def test_nan_and_signs():
    assert oracle.fill_bits(float("nan"), "float32") == 0x7FC00000
    assert oracle.fill_bits(-float("nan"), "bfloat16") == 0xFFC0
    assert oracle.fill_bits(-0.0, "float16") == 0x8000
    assert oracle.fill_bits(0.0, "float32") == 0
