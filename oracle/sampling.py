"""CPU oracle for token sampling after the LM head (float64 NumPy).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Follows the lab page's ``sample`` function and chapter 5's filter-and-sample
listing, in their order: temperature, then top-k, then top-p (nucleus), then
renormalise and draw. Serving tutorial demos D01/D02 fix the corner cases:
greedy (temperature 0) takes the lowest index among tied maxima; top-k keeps
exactly k tokens; top-p keeps the shortest prefix of the descending order
whose cumulative mass reaches p, boundary token included; adding a
constant to the logits changes no support; top-k then top-p differs from
top-p then top-k.

Readings where the pages are silent: scaled logits are ``logit / T`` in
float32 (the device's precision; comparisons of scaled logits are then the
same on both sides); ties in the descending order go to the lower index;
the draw is the inverse CDF of the kept probabilities in vocabulary order
(``rng.choice(VOCAB, p=filtered)`` in the lab), with the uniform number
passed in: the token is the first index whose cumulative kept mass exceeds
``u`` times the total.
"""
from __future__ import annotations

import numpy as np


def scaled_logits(logits, temperature) -> np.ndarray:
    """``logit / T`` rounded to float32 (T > 0)."""
    if not temperature > 0:
        raise ValueError("temperature must be positive (0 selects greedy decoding)")
    return (np.asarray(logits, dtype=np.float32) / np.float32(temperature)).astype(np.float64)


def desc_order(values) -> np.ndarray:
    """Indices by decreasing value, ties by increasing index."""
    v = np.asarray(values)
    return np.lexsort((np.arange(len(v)), -v))


def greedy(logits) -> int:
    """argmax, lowest index among ties (demo D01)."""
    return int(desc_order(np.asarray(logits, dtype=np.float64))[0])


def top_k_filter(probs, k: int) -> np.ndarray:
    """Zero all but the k largest probabilities (ties by lower index); k <= 0
    or k >= len keeps everything. Returns the kept (unnormalised) masses."""
    p = np.asarray(probs, dtype=np.float64)
    if k <= 0 or k >= len(p):
        return p.copy()
    out = np.zeros_like(p)
    keep = desc_order(p)[:k]
    out[keep] = p[keep]
    return out


def top_p_filter(probs, top_p: float) -> np.ndarray:
    """Keep the shortest prefix of the descending order whose cumulative
    share of the total reaches ``top_p`` (boundary token kept; the largest is
    always kept): token j stays iff the share strictly before it is below
    ``top_p``. ``top_p >= 1`` keeps everything."""
    p = np.asarray(probs, dtype=np.float64)
    if top_p >= 1.0:
        return p.copy()
    order = desc_order(p)
    total = p.sum()
    before = np.concatenate([[0.0], np.cumsum(p[order])[:-1]])
    keep = order[(before < top_p * total) | (np.arange(len(p)) == 0)]
    out = np.zeros_like(p)
    out[keep] = p[keep]
    return out


def sample(logits, temperature: float, top_k: int, top_p: float, u: float):
    """Returns ``(token, kept_after_top_k, kept_after_top_p, filtered)``.

    Chapter 5's listing: scaled logits sorted in decreasing order (ties: lower
    index), top-k keeps the first k of that order, masses ``exp(z - max z)``,
    top-p keeps the prefix whose share strictly before each token is below
    ``top_p`` (the first always), then the lab's draw in vocabulary order.
    ``filtered`` are the kept masses (unnormalised)."""
    if temperature == 0:
        t = greedy(logits)
        f = np.zeros(len(logits))
        f[t] = 1.0
        return t, 1, 1, f
    z = scaled_logits(logits, temperature)
    V = len(z)
    order = desc_order(z)
    keep = order if (top_k <= 0 or top_k >= V) else order[:top_k]
    mass = np.exp(z[keep] - z.max())
    if top_p < 1.0:
        before = np.concatenate([[0.0], np.cumsum(mass)[:-1]])
        stay = (before < top_p * mass.sum())
        stay[0] = True
        kept_p, mass_p = keep[stay], mass[stay]
    else:
        kept_p, mass_p = keep, mass
    pp = np.zeros(V)
    pp[kept_p] = mass_p
    cdf = np.cumsum(pp)
    token = int(np.searchsorted(cdf, u * cdf[-1], side="right"))
    token = min(token, int(kept_p.max()))
    return token, len(keep), len(kept_p), pp


def cdf_margin(filtered, u: float, token: int) -> float:
    """Distance (as a share of the total) from ``u`` to the nearer edge of the
    drawn token's CDF step; near 0 the draw is decided by rounding."""
    cdf = np.cumsum(filtered) / filtered.sum()
    lo = cdf[token - 1] if token > 0 else 0.0
    return float(min(u - lo, cdf[token] - u))
