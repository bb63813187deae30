"""Pins for the sampler oracle (oracle/sampler.py).

* Philox4x32-10 against the published known-answer vectors;
* the uniform conversion is exact and strictly inside (0, 1);
* keep sets and greedy picks worked by hand (tests/golden/sampler_cases.json);
* draws: determinism in (seed, offset), sensitivity to the offset, masked
  tokens never drawn, and a chi-square test of the draw distribution against
  the renormalised filtered softmax -- which also catches a wrong Gumbel
  transform (planted mistakes below must fail it).
"""

import json
import math
import pathlib

import numpy as np
import pytest

from oracle import sampler as S

GOLD = pathlib.Path(__file__).resolve().parent / "golden"
KAT = json.loads((GOLD / "philox4x32_kat.json").read_text())["cases"]
CASES = json.loads((GOLD / "sampler_cases.json").read_text())


@pytest.mark.parametrize("case", KAT)
def test_philox_known_answers(case):
    c = [np.uint64(int(x, 16)) for x in case["counter"]]
    k = [np.uint64(int(x, 16)) for x in case["key"]]
    out = S.philox4x32(*c, *k)
    assert [int(o) for o in out] == [int(x, 16) for x in case["out"]]


@pytest.mark.parametrize("case", KAT)
def test_uniforms_word_order_against_known_answers(case):
    """Token i of a row reads word i % 4 of the Philox block for counter
    (i // 4, row, offset low, offset high) under key (seed low, seed high):
    each published vector, read through that placement, gives the four
    tokens' words, in order."""
    c = [int(x, 16) for x in case["counter"]]
    k = [int(x, 16) for x in case["key"]]
    want = [int(x, 16) for x in case["out"]]
    u = S.uniforms(seed=k[0] | (k[1] << 32), offset=c[2] | (c[3] << 32), row=c[1], n=4, first=4 * c[0])
    assert u.tolist() == [((w >> 9) + 0.5) / (1 << 23) for w in want]


def test_uniforms_exact_and_open_interval():
    u = S.uniforms(seed=123, offset=7, row=3, n=100000)
    assert (u > 0).all() and (u < 1).all()
    scaled = u * (1 << 23) - 0.5
    assert np.array_equal(scaled, np.floor(scaled))
    assert np.array_equal(u.astype(np.float32).astype(np.float64), u)     # exact in binary32
    assert abs(u.mean() - 0.5) < 0.01


@pytest.mark.parametrize("case", CASES["cases"], ids=[str(i) for i in range(len(CASES["cases"]))])
def test_keep_sets_by_hand(case):
    z = np.array(case["logits"], dtype=np.float64)
    cut = S.keep_threshold(z, np.ones(z.size, bool), case["top_k"], case["top_p"], case["min_p"])
    assert np.flatnonzero(z >= cut).tolist() == case["keep"]
    p = S.filtered_probs(z, np.ones(z.size, bool), 1.0, case["top_k"], case["top_p"], case["min_p"])
    assert np.flatnonzero(p > 0).tolist() == case["keep"]
    assert math.isclose(p.sum(), 1.0)


@pytest.mark.parametrize("case", CASES["greedy"])
def test_greedy_by_hand(case):
    z = np.array(case["logits"], dtype=np.float64)
    tok, _ = S.sample_row(z, np.ones(z.size, bool), 0.0, 0, 1.0, 0.0, 0, 0, 0)
    assert tok == case["token"]


def draws(logits, allowed, T, k, p, m, n, seed=5, row=0):
    return np.array([S.sample_row(logits, allowed, T, k, p, m, seed, off, row)[0] for off in range(n)])


def test_determinism_and_offsets():
    rng = np.random.default_rng(1)
    z = rng.standard_normal(300) * 2
    a = np.ones(300, bool)
    t1 = draws(z, a, 1.0, 0, 1.0, 0.0, 200)
    t2 = draws(z, a, 1.0, 0, 1.0, 0.0, 200)
    assert np.array_equal(t1, t2)
    assert len(set(t1.tolist())) > 50                 # offsets change the draw
    other_row = np.array([S.sample_row(z, a, 1.0, 0, 1.0, 0.0, 5, off, 1)[0] for off in range(200)])
    assert (other_row != t1).mean() > 0.8             # rows are independent streams


def test_masked_tokens_never_drawn():
    rng = np.random.default_rng(2)
    z = rng.standard_normal(64) * 3
    mask_row = np.array([0x0F0F00F0, 0x00000001], dtype=np.uint32).view(np.int32)
    allowed = S.allowed_tokens(mask_row, 64, 64)
    assert np.flatnonzero(allowed).tolist() == [4, 5, 6, 7, 16, 17, 18, 19, 24, 25, 26, 27, 32]
    t = draws(z, allowed, 0.8, 0, 1.0, 0.0, 500)
    assert set(t.tolist()) <= set(np.flatnonzero(allowed).tolist())
    assert S.sample_row(z, np.zeros(64, bool), 1.0, 0, 1.0, 0.0, 0, 0, 0)[0] == -1


def chi_square_ok(tokens, probs, min_expected=5.0):
    n = tokens.size
    counts = np.bincount(tokens, minlength=probs.size)
    if (counts[probs == 0] > 0).any():
        return False
    exp = probs * n
    big = exp >= min_expected
    stat = (((counts[big] - exp[big]) ** 2) / exp[big]).sum()
    rest_o, rest_e = counts[~big & (probs > 0)].sum(), exp[~big & (probs > 0)].sum()
    if rest_e > 0:
        stat += (rest_o - rest_e) ** 2 / rest_e
    dof = int(big.sum()) + (1 if rest_e > 0 else 0) - 1
    # chi-square tail bound via Wilson-Hilferty: accept below the 1e-6 quantile region
    zscore = ((stat / dof) ** (1 / 3) - (1 - 2 / (9 * dof))) / math.sqrt(2 / (9 * dof))
    return zscore < 4.75


@pytest.mark.parametrize("T,k,p,m", [(1.0, 0, 1.0, 0.0), (0.7, 8, 1.0, 0.0), (1.3, 0, 0.8, 0.0),
                                      (1.0, 0, 1.0, 0.05), (0.9, 12, 0.9, 0.02)])
def test_draw_distribution(T, k, p, m):
    rng = np.random.default_rng(3)
    z = rng.standard_normal(40) * 1.5
    a = np.ones(40, bool)
    a[[3, 17]] = False
    t = draws(z, a, T, k, p, m, 8000)
    assert chi_square_ok(t, S.filtered_probs(z, a, T, k, p, m))


MUTANT_GUMBELS = {
    "exponential variates": lambda u: -np.log(u),
    "sign flipped": lambda u: np.log(-np.log(u)),
    "raw uniforms": lambda u: u,
}


@pytest.mark.parametrize("name", list(MUTANT_GUMBELS))
def test_planted_gumbel_mistakes_fail_distribution(name, monkeypatch):
    rng = np.random.default_rng(4)
    z = rng.standard_normal(30) * 2.0
    a = np.ones(30, bool)
    probs = S.filtered_probs(z, a, 1.0, 0, 1.0, 0.0)
    assert chi_square_ok(draws(z, a, 1.0, 0, 1.0, 0.0, 6000), probs)
    monkeypatch.setattr(S, "gumbel", MUTANT_GUMBELS[name])
    assert not chi_square_ok(draws(z, a, 1.0, 0, 1.0, 0.0, 6000), probs)


def test_non_positive_temperature_and_top_p_edges():
    """Readings where the page is silent, pinned against direct definitions:
    a temperature that is not positive (0, negative, NaN) is the argmax of
    the allowed finite logits (lowest index on ties); top-p with p <= 0 keeps
    exactly the tokens equal to the largest allowed logit."""
    rng = np.random.default_rng(31)
    x = np.round(rng.standard_normal(200) * 2, 1)            # many ties
    allowed = rng.random(200) < 0.5
    best = np.max(x[allowed])
    argmax = int(np.flatnonzero(allowed & (x == best))[0])
    for T in (0.0, -1.0, float("nan")):
        tok, _ = S.sample_row(x, allowed, T, 0, 1.0, 0.0, 1, 2, 0)
        assert tok == argmax
    for p in (0.0, -0.5, -math.inf):
        cut = S.keep_threshold(x, allowed, 0, p, 0.0)
        assert cut == best
        keep = allowed & (x >= cut)
        assert np.array_equal(keep, allowed & (x == best))


def test_min_p_at_or_above_one_and_infinite_temperature():
    """min_p >= 1 keeps exactly the tokens equal to the largest allowed logit
    (no filter empties a set that has a candidate); an infinite temperature
    makes every z equal, so top-k, top-p and min-p keep every allowed token
    and the draw is the argmax of the Gumbel variates alone."""
    rng = np.random.default_rng(32)
    x = np.round(rng.standard_normal(300) * 2, 1)
    allowed = rng.random(300) < 0.5
    best = np.max(x[allowed])
    for m in (1.0, 1.5, math.inf):
        cut = S.keep_threshold(x, allowed, 0, 1.0, m)
        assert np.array_equal(allowed & (x >= cut), allowed & (x == best))
    z = x / math.inf
    cut = S.keep_threshold(z, allowed, 3, 0.5, 0.9)
    assert np.array_equal(allowed & (z >= cut), allowed)
    tok, _ = S.sample_row(x, allowed, math.inf, 3, 0.5, 0.9, 4, 5, 6)
    g = S.gumbel(S.uniforms(4, 5, 6, 300))
    assert tok == int(np.flatnonzero(allowed)[np.argmax(g[allowed])])
