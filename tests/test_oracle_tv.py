"""Pins for the TV bound (oracle/tv.py).

What pins it:
* TV is a distance: 0 on equal inputs, symmetric, 1 on disjoint supports;
* brute force over every +-E sign pattern on small softmaxes never exceeds
  tanh(E/2), and the closed-form worst case (mass 1/(1+e^E) moved up, the
  rest down) attains it; random perturbations inside the box stay below it;
* tanh(E/2) <= tanh(E), the pages' prior form;
* on INT8 caches, the true TV between exact-key and quantized-key weights is
  below tanh(cmax/2), also for a block made coarse by an outlier key.
"""

import numpy as np
import pytest

from oracle import tv
from oracle.attention import softmax_weights


def test_tv_distance_axioms():
    p = np.array([0.2, 0.3, 0.5])
    assert tv.tv_distance(p, p) == 0.0
    q = np.array([0.5, 0.3, 0.2])
    assert tv.tv_distance(p, q) == tv.tv_distance(q, p) == pytest.approx(0.3)
    assert tv.tv_distance([1, 0], [0, 1]) == 1.0


@pytest.mark.parametrize("n", [2, 3, 4, 6])
def test_sign_patterns_never_exceed_tanh_half(n):
    rng = np.random.default_rng(n)
    for _ in range(40):
        p = rng.dirichlet(np.ones(n) * rng.uniform(0.2, 3))
        p = np.clip(p, 1e-12, None)
        p /= p.sum()
        e = rng.uniform(0.001, 3.0)
        assert tv.max_tv_over_signs(p, e) <= tv.tv_bound(e) + 1e-12


def test_worst_case_attains_the_bound():
    for e in [0.01, 0.3, 1.0, 2.5]:
        a = 1.0 / (1.0 + np.exp(e))
        p = np.array([a, 1 - a])
        pert = softmax_weights(np.log(p) + np.array([e, -e]))
        assert tv.tv_distance(p, pert) == pytest.approx(np.tanh(e / 2), rel=1e-12)
        assert tv.max_tv_over_signs(p, e) == pytest.approx(np.tanh(e / 2), rel=1e-12)


def test_random_perturbations_inside_the_box():
    rng = np.random.default_rng(1)
    for _ in range(300):
        n = int(rng.integers(2, 40))
        s = rng.standard_normal(n) * rng.uniform(0.1, 5)
        e = rng.uniform(0.0, 2.0)
        eps = rng.uniform(-e, e, n)
        t = tv.tv_distance(softmax_weights(s), softmax_weights(s + eps))
        assert t <= tv.tv_bound(e) + 1e-12
        assert tv.tv_bound(e) <= tv.prior_tv_bound(e)


def test_int8_cache_tv_below_bound():
    rng = np.random.default_rng(2)
    d, w = 128, 64
    for n in [5, 16, 40, 64, 100]:
        k, v = rng.standard_normal((n, d)), rng.standard_normal((n, d))
        k = k.astype(np.float32).astype(np.float64)
        q = rng.standard_normal(d) * 3
        r = tv.int8_attention_tv(q, k, v, n, w)
        assert r["tv"] <= r["bound"]
        assert r["cmax"] >= r["emax"]
    # an outlier key makes its block's scale coarse: larger error, still bounded
    k = rng.standard_normal((48, d))
    k[20, 7] = 400.0
    q = rng.standard_normal(d) * 3
    r = tv.int8_attention_tv(q, k, rng.standard_normal((48, d)), 48, 64)
    assert r["tv"] <= r["bound"] and r["bound"] > 0.2


def test_bound_is_attained_by_tv_bound():
    for e in [0.05, 0.7, 2.0]:
        a = 1.0 / (1.0 + np.exp(e))
        assert tv.max_tv_over_signs(np.array([a, 1 - a]), e) == pytest.approx(tv.tv_bound(e), rel=1e-12)


def test_int8_tv_via_one_hot_values():
    """With value rows a*e_j (one-hot, a = 127/128 so the block scale 2^-7 and
    the codes are exact), attention returns a times its weight vector, so the
    INT8 decode output and the masked float64 attention give the
    quantized-key and exact-key weights by another route."""
    from oracle import attention, int8 as oint8
    rng = np.random.default_rng(4)
    d, w = 128, 64
    for n in [40, 64, 100]:
        k = rng.standard_normal((n, d)).astype(np.float32).astype(np.float64)
        q = rng.standard_normal(d) * 2
        v = np.zeros((n, d))
        ln = min(w, n)
        for i, p in enumerate(range(n - ln, n)):
            v[p, i] = 127.0 / 128.0
        pq = oint8.int8_decode(q, k, v, n, w)["out"][:ln] / (127.0 / 128.0)
        pe = attention.masked_attention(q, np.arange(n), k, v, n - 1, w)[:ln] / (127.0 / 128.0)
        r = tv.int8_attention_tv(q, k, v, n, w)
        assert r["tv"] == pytest.approx(tv.tv_distance(pe, pq), abs=1e-12)
        assert r["tv"] > 0


def test_empty_history_has_zero_tv_and_bound():
    """Nothing visible: no attention weights move, so TV and bound are 0."""
    d = 128
    z = np.zeros((0, d))
    r = tv.int8_attention_tv(np.ones(d), z, z, 0, 64)
    assert r["tv"] == 0.0 and r["bound"] == 0.0 and r["cmax"] == 0.0


@pytest.mark.parametrize("p0", [0.1, 0.9, 0.5, 0.02])
def test_two_token_worst_case_in_closed_form(p0):
    """Two tokens: the sign patterns that move anything raise one logit by e
    and lower the other by e, which multiplies that token's odds by e^(2e);
    the largest TV over sign patterns is the larger of the two closed forms
    p' - p with p' = p e^(2e) / (p e^(2e) + 1 - p), whichever token it is."""
    e = 0.7
    p = np.array([p0, 1 - p0])
    want = max(pi * np.exp(2 * e) / (pi * np.exp(2 * e) + 1 - pi) - pi for pi in p)
    assert tv.max_tv_over_signs(p, e) == pytest.approx(want, rel=1e-12)
