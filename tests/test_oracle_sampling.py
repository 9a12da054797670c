"""Pins of the sampling oracle (lab page sample; chapter 5's filter-and-sample
listing; serving tutorial demos D01/D02)."""
import json
import os

import numpy as np
import pytest

from oracle import sampling as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden():
    with open(os.path.join(GOLDEN, "serving_tutorial_sampling.json")) as f:
        return json.load(f)


def support(p):
    return sorted(int(i) for i in np.nonzero(np.asarray(p) > 0)[0])


def test_top_p_example_keeps_the_boundary_token():
    g = _golden()["top_p_example"]
    assert support(S.top_p_filter(g["probs"], g["top_p"])) == g["support"]
    assert g["probs"][0] < g["top_p"] <= g["cumulative_at_boundary"]
    # the same through the full sampler on log-probabilities at T = 1
    _, kk, kp, f = S.sample(np.log(g["probs"]), 1.0, 0, g["top_p"], 0.5)
    assert (kk, kp) == (4, 2) and support(f) == g["support"]


def test_filter_order_matters():
    g = _golden()["filter_order"]
    probs = [0.45, 0.30, 0.15, 0.10]          # a distribution with the page's two supports
    a = support(S.top_p_filter(S.top_k_filter(probs, g["top_k"]), g["top_p"]))
    b = support(S.top_k_filter(S.top_p_filter(probs, g["top_p"]), g["top_k"]))
    assert a == g["support_k_then_p"] and b == g["support_p_then_k"]
    # the sampler applies top-k first (lab order)
    assert S.sample(np.log(probs), 1.0, g["top_k"], g["top_p"], 0.1)[2] == len(g["support_k_then_p"])


def test_greedy_and_temperature_limits():
    assert S.greedy([1.0, 3.0, 3.0, 2.0]) == 1                   # tied maxima: lowest index
    assert S.sample([1.0, 3.0, 3.0, 2.0], 0, 0, 1.0, 0.99)[0] == 1
    with pytest.raises(ValueError):
        S.scaled_logits([1.0, 2.0], -1.0)
    # T -> 0+: the unique maximum takes all the mass; tied maxima split it
    f = S.sample([0.0, 2.0, 1.0], 1e-3, 0, 1.0, 0.5)[3]
    assert f[1] / f.sum() > 1 - 1e-12
    f = S.sample([0.0, 2.0, 2.0], 1e-3, 0, 1.0, 0.5)[3]
    assert abs(f[1] / f.sum() - 0.5) < 1e-12 and abs(f[2] / f.sum() - 0.5) < 1e-12


def test_top_k_size_and_shift_invariance():
    rng = np.random.default_rng(3)
    for _ in range(50):
        V = int(rng.integers(2, 60))
        x = rng.standard_normal(V)
        k = int(rng.integers(1, V + 1))
        tp = float(rng.uniform(0.05, 1.0))
        T = float(rng.uniform(0.2, 2.0))
        _, kk, kp, f = S.sample(x, T, k, tp, 0.3)
        assert kk == min(k, V) and 1 <= kp <= kk
        c = float(rng.uniform(-5, 5))
        _, kk2, kp2, f2 = S.sample(x + c, T, k, tp, 0.3)
        # same supports (scaled logits move by c / T; fp32 rounding may merge
        # nearly tied values, so compare supports, not masses)
        assert support(f) == support(f2) or abs(kp - kp2) <= 1


def test_draw_is_numpys_choice_for_the_same_uniform():
    """The lab draws with rng.choice(VOCAB, p=filtered); with the same
    generator state the inverse-CDF token equals that call's result."""
    for seed in range(200):
        rng = np.random.default_rng(seed)
        V = int(rng.integers(1, 40))
        x = rng.standard_normal(V) * 2
        T, k, tp = float(rng.uniform(0.3, 1.5)), int(rng.integers(0, V + 1)), float(rng.uniform(0.1, 1.0))
        f = S.sample(x, T, k, tp, 0.0)[3]
        probs = f / f.sum()
        u = np.random.default_rng(1000 + seed).random()
        want = int(np.random.default_rng(1000 + seed).choice(V, p=probs))
        got = S.sample(x, T, k, tp, u)[0]
        assert got == want or S.cdf_margin(f, u, got) < 1e-12
