"""CPU oracle for the fused bitmask-apply + sampler.

TEST INFRASTRUCTURE, like the rest of ``oracle/``: only tests, the smoke
check and the bench's CPU-baseline leg use it.

What it follows (logits-processor page, "Ops: sample" and "How it works"):

* per-row temperature: z = logit / T; T <= 0 means greedy (argmax);
* three filters, each keeping the largest-probability tokens above a cutoff,
  so their intersection is one threshold (no sort needed):
    top-k  (k <= 0 disables): keep tokens whose probability is at least the
           k-th largest one;
    top-p  (p >= 1 disables): keep tokens whose probability is at least the
           largest cutoff t for which the tokens at or above t hold at least
           a fraction p of the mass (the nucleus);
    min-p  (m <= 0 disables): keep tokens whose probability is at least m
           times the largest one;
  ties at a cutoff are kept (a threshold, not a count);
* the draw: one token from the kept set with probability proportional to its
  softmax probability, by Gumbel-max (argmax of log-probability plus an
  independent Gumbel variate per token);
* the variates come from a counter-based generator keyed by (seed, row,
  offset): the same (seed, offset) replays the same tokens.
* with a bitmask, masked tokens (and tokens at or past the vocab size) take
  no part, so a masked token is never drawn (logits-processor page,
  Correctness: a bitmask followed by sample never draws a disallowed token).

Readings where the page is silent:

* generator: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random
  Numbers: As Easy as 1, 2, 3", SC 2011), written here from its definition:
  key = (seed low 32 bits, seed high 32 bits); for token i of row r the
  counter is (i // 4, r, offset low, offset high) and word i % 4 is used;
* uniform: u = (floor(x / 2^9) + 1/2) / 2^23 for the 32-bit word x, so
  0 < u < 1 and u is exact in binary32 (24 significant bits);
* Gumbel variate: g = -ln(-ln(u));
* greedy and Gumbel-max ties go to the lowest token index;
* a temperature that is not positive -- NaN included -- is greedy; top-p
  with p <= 0 keeps only the largest value and its ties (any mass reaches
  p), as p = 0 does, and so does min-p with m >= 1 (no filter empties a set
  that has a candidate);
* a row with no allowed token draws -1; a logit that is not finite (-inf
  from an earlier mask, +inf, NaN) counts as not allowed.

Everything is float64 except the generator (exact integers).
"""

from __future__ import annotations

import math
from typing import Optional

import numpy as np

M0, M1 = 0xD2511F53, 0xCD9E8D57      # Philox4x32 multipliers
W0, W1 = 0x9E3779B9, 0xBB67AE85      # Weyl key increments
MASK32 = 0xFFFFFFFF


def philox4x32(c0, c1, c2, c3, k0, k1, rounds: int = 10):
    """Philox4x32-R on numpy uint64 arrays holding 32-bit values (vectorised).

    Each round: multiply counter words 0 and 2 by the two constants (full
    64-bit products), then the new counter is (hi(M1*c2) ^ c1 ^ k0,
    lo(M1*c2), hi(M0*c0) ^ c3 ^ k1, lo(M0*c0)); the key advances by the Weyl
    constants between rounds.
    """
    c0, c1, c2, c3 = (np.asarray(x, dtype=np.uint64) & MASK32 for x in (c0, c1, c2, c3))
    k0 = np.asarray(k0, dtype=np.uint64) & MASK32
    k1 = np.asarray(k1, dtype=np.uint64) & MASK32
    for r in range(rounds):
        if r:
            k0 = (k0 + W0) & MASK32
            k1 = (k1 + W1) & MASK32
        p0 = c0 * np.uint64(M0)
        p1 = c2 * np.uint64(M1)
        hi0, lo0 = p0 >> np.uint64(32), p0 & np.uint64(MASK32)
        hi1, lo1 = p1 >> np.uint64(32), p1 & np.uint64(MASK32)
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def uniforms(seed: int, offset: int, row: int, n: int, first: int = 0) -> np.ndarray:
    """float64 u in (0, 1) for tokens first..first+n-1 of one row (exact binary32 values).

    Token i takes word i % 4 of the block for counter (i // 4, row, offset
    low, offset high) under key (seed low, seed high).
    """
    i = np.arange(first, first + n, dtype=np.uint64)
    words = philox4x32(i >> np.uint64(2), np.uint64(row), np.uint64(offset & MASK32),
                       np.uint64((offset >> 32) & MASK32), np.uint64(seed & MASK32),
                       np.uint64((seed >> 32) & MASK32))
    x = np.choose((i & np.uint64(3)).astype(np.int64), words)
    return ((x >> np.uint64(9)).astype(np.float64) + 0.5) / float(1 << 23)


def gumbel(u: np.ndarray) -> np.ndarray:
    """Standard Gumbel variates from uniforms: -ln(-ln u)."""
    return -np.log(-np.log(u))


def keep_threshold(z: np.ndarray, allowed: np.ndarray, top_k: int, top_p: float, min_p: float) -> float:
    """The smallest kept z (all filters intersected); z is float64, masked tokens excluded."""
    za = z[allowed]
    zmax = za.max()
    probs = np.exp(za - zmax)
    probs /= probs.sum()
    cut = -math.inf
    if top_k > 0 and top_k < za.size:
        cut = max(cut, np.sort(za)[::-1][top_k - 1])
    if top_p < 1.0:
        # distinct values in descending order, and the mass at or above each
        values = np.unique(za)[::-1]
        order = np.argsort(-za, kind="stable")
        cum = np.cumsum(probs[order])
        sorted_z = za[order]
        # last position (in descending order) holding each distinct value
        last = np.searchsorted(-sorted_z, -values, side="right") - 1
        mass_at_or_above = cum[last]
        reach = np.flatnonzero(mass_at_or_above >= top_p)
        cut = max(cut, values[reach[0]] if reach.size else values[-1])
    if min_p > 0.0:
        # the cut never passes the largest value: min_p >= 1 keeps it and its ties
        cut = max(cut, zmax + min(math.log(min_p), 0.0))
    return cut


def sample_row(logits: np.ndarray, allowed: np.ndarray, temperature: float, top_k: int, top_p: float,
               min_p: float, seed: int, offset: int, row: int, margin: float = 0.0):
    """(token, details) for one row.

    ``logits`` float64 [V], ``allowed`` bool [V].  ``details`` holds the keep
    set, the Gumbel keys and, with ``margin`` > 0, the set of tokens a float32
    implementation may legitimately return: winners over keep sets loosened
    and tightened by ``margin`` (relative, in probability) and any kept token
    whose key is within ``margin`` of the best.
    """
    V = logits.size
    allowed = allowed & np.isfinite(logits)
    if not allowed.any():
        return -1, {"keep": np.zeros(V, bool), "candidates": {-1}}
    if not temperature > 0.0:  # T <= 0, or NaN: greedy
        best = np.max(logits[allowed])
        token = int(np.flatnonzero(allowed & (logits == best))[0])
        return token, {"keep": allowed & (logits == best), "candidates": {token}}
    z = logits / temperature
    cut = keep_threshold(z, allowed, top_k, top_p, min_p)
    keep = allowed & (z >= cut)
    u = uniforms(seed, offset, row, V)
    key = np.full(V, -math.inf)
    g = gumbel(u)
    key[keep] = z[keep] + g[keep]
    token = int(np.argmax(key))
    cands = {token}
    if margin > 0.0:
        for c in (cut + math.log1p(-margin), cut + math.log1p(margin)):
            k2 = allowed & (z >= c)
            if k2.any():
                key2 = np.where(k2, z + g, -math.inf)
                cands.add(int(np.argmax(key2)))
        loose = allowed & (z >= cut + math.log1p(-margin))
        key3 = np.where(loose, z + g, -math.inf)
        cands |= set(np.flatnonzero(key3 >= key3.max() - margin).tolist())
    return token, {"keep": keep, "cut": cut, "key": key, "candidates": cands}


def filtered_probs(logits: np.ndarray, allowed: np.ndarray, temperature: float, top_k: int, top_p: float,
                   min_p: float) -> np.ndarray:
    """The renormalised softmax over the kept set (the distribution of a draw)."""
    allowed = allowed & np.isfinite(logits)
    out = np.zeros(logits.size)
    if not allowed.any():
        return out
    if not temperature > 0.0:  # T <= 0, or NaN: greedy
        best = np.max(logits[allowed])
        out[int(np.flatnonzero(allowed & (logits == best))[0])] = 1.0
        return out
    z = logits / temperature
    keep = allowed & (z >= keep_threshold(z, allowed, top_k, top_p, min_p))
    w = np.where(keep, np.exp(z - z[keep].max()), 0.0)
    return w / w.sum()


def allowed_tokens(mask_row: Optional[np.ndarray], vocab_size: int, cols: int) -> np.ndarray:
    """bool [cols]: token v < vocab_size whose bit v % 32 of word v // 32 is set (all, without a mask)."""
    out = np.zeros(cols, dtype=bool)
    if mask_row is None:
        out[:vocab_size] = True
        return out
    v = np.arange(vocab_size)
    words = (mask_row.astype(np.int64) & MASK32)[v // 32]
    out[:vocab_size] = ((words >> (v % 32)) & 1).astype(bool)
    return out
