"""Pins of the joint-vs-marginal facts (Fast-dLLM reading notes secs. 4-5.2;
decoding-and-speed page, parallel-decoding section) by printed values and
brute force over tiny vocabularies."""
import json
import os

import numpy as np
import pytest

from oracle import theory as T
from oracle.sampler import select_threshold

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def test_two_position_example_printed_values():
    g = _gold("two_position_example.json")
    p = np.array(g["joint"])
    m = T.marginals(p)
    assert np.allclose([m[0][0], m[1][0]], g["marginal_top"], atol=1e-12)
    q = T.product_of_marginals(p)
    assert np.allclose(q, np.array(g["product"]), atol=1e-12)
    assert abs(T.tv(p, q) - g["tv"]) < 1e-12
    # greedy per-position choice is (0,0) while the joint prefers (0,1)/(1,0)
    assert T.greedy_marginal_choice(p) == (0, 0)
    assert set(T.argmax_set(p)) == {(0, 1), (1, 0)}
    assert T.kl(q, p) == float("inf")


def test_forward_kl_is_total_correlation_two_ways():
    # eq. 11: KL(p||q) = sum H(X_j) - H(X) = sum_j I(X_j; X_<j)
    rng = np.random.default_rng(0)
    for n, V in [(2, 2), (3, 3), (4, 2)]:
        p = rng.random((V,) * n)
        p /= p.sum()
        q = T.product_of_marginals(p)
        kl = T.kl(p, q)
        assert abs(kl - T.total_correlation(p)) < 1e-12
        # chain rule: sum_j [H(X_j) + H(X_<j) - H(X_<=j)]
        chain = 0.0
        for j in range(1, n):
            pj = p.sum(axis=tuple(range(j + 1, n)))           # X_1..X_{j+1}
            prev = pj.sum(axis=j)
            xj = pj.sum(axis=tuple(range(j)))
            chain += T.entropy(xj) + T.entropy(prev) - T.entropy(pj)
        assert abs(kl - chain) < 1e-12
    g = _gold("two_position_example.json")
    p = np.array(g["joint"])
    # closed form for the example: 2 H(0.66) - H(.32,.34,.34)
    h = lambda *a: -sum(x * np.log(x) for x in a if x > 0)
    assert abs(T.kl(p, T.product_of_marginals(p)) - (2 * h(0.66, 0.34) - h(0.32, 0.34, 0.34))) < 1e-12


def test_poker_example():
    g = _gold("poker_example.json")
    # positions: (full|high), (house|card); half full house, half high card
    p = np.array([[0.5, 0.0], [0.0, 0.5]])
    q = T.product_of_marginals(p)
    assert np.allclose([m.max() for m in T.marginals(p)], g["marginal"])
    assert abs(q[0, 0] + q[1, 1] - g["valid_prob_one_step"]) < 1e-12
    assert (g["n"] + 1) * g["eps"] == g["premise_lhs"]
    assert not T.theorem1_premise(p, g["eps"])
    # the threshold rule (tau 0.9) commits one position first (fallback)
    sel = select_threshold(np.array([0.5, 0.5], np.float32), np.array([0, 1]), 0.9)
    assert len(sel) == 1
    t = g["three_positions_at_0_95"]
    assert abs((t["n"] + 1) * t["eps"] - t["premise_lhs"]) < 1e-12 and (t["n"] + 1) * t["eps"] <= 1


def _concentrated_joint(rng, n, V, eps):
    """Random joint whose every marginal puts > 1-eps on a random x*."""
    xs = tuple(int(v) for v in rng.integers(0, V, n))
    for _ in range(1000):
        noise = rng.random((V,) * n) ** 4
        noise /= noise.sum()
        delta = rng.random() * eps * 0.999
        p = delta * noise
        p[xs] += 1 - delta
        if all(m.max() > 1 - eps for m in T.marginals(p)):
            return p, xs
    raise RuntimeError


@pytest.mark.parametrize("n,V", [(2, 2), (2, 4), (3, 3), (4, 2), (5, 2)])
def test_theorem1_brute_force(n, V):
    rng = np.random.default_rng(n * 10 + V)
    eps = 1.0 / (n + 1)
    for _ in range(300):
        p, xs = _concentrated_joint(rng, n, V, eps * rng.random() ** 0.3)
        e = max(1 - m.max() for m in T.marginals(p)) + 1e-15
        assert T.theorem1_premise(p, e)
        q = T.product_of_marginals(p)
        assert T.argmax_set(p) == [xs]
        assert T.argmax_set(q) == [xs]


@pytest.mark.parametrize("n", [2, 3, 4, 5, 6])
def test_tightness_construction(n):
    for eta in (1e-3, 1e-2):
        p = T.tightness_joint(n, eta)
        assert abs(p.sum() - 1) < 1e-12
        m = T.marginals(p)
        # every marginal prefers 0 ...
        assert all(mj[0] > mj[1] for mj in m)
        # ... yet the joint argmax is a single-1 string, not all zeros
        am = T.argmax_set(p)
        assert (0,) * n not in am and all(sum(s) == 1 for s in am)
        # the premise fails, just barely: eps = 1/(n+1) + eta/n
        e = 1 - min(mj[0] for mj in m)
        assert abs(e - (1.0 / (n + 1) + eta / n)) < 1e-12
        assert (n + 1) * e > 1
    # confidence boundary n/(n+1) (reading notes Fig. 3 description)
    assert abs(1 - 1.0 / (n + 1) - n / (n + 1)) < 1e-15


@pytest.mark.parametrize("n,V", [(2, 3), (3, 2), (3, 3), (4, 2)])
def test_tv_lr_kl_bounds(n, V):
    rng = np.random.default_rng(7 * n + V)
    for _ in range(200):
        eps = rng.random() / (n + 1)
        p, _ = _concentrated_joint(rng, n, V, eps)
        e = max(1 - m.max() for m in T.marginals(p))
        q = T.product_of_marginals(p)
        assert T.tv(p, q) < T.tv_bound(n, e) + 1e-15
        for r in (1.0, 2.0, 3.0):
            assert T.lr_norm(p, q, r) < T.lr_bound(n, e, r) + 1e-15
        assert T.kl(p, q) < T.kl_bound(n, e, V) + 1e-15


def test_nonuniform_budget_brute_force():
    # eq. 9: sum eps_j + max eps_j < 1  =>  x* is the joint argmax
    rng = np.random.default_rng(3)
    hits = 0
    for _ in range(2000):
        n, V = int(rng.integers(2, 5)), int(rng.integers(2, 4))
        p = rng.random((V,) * n) ** 8
        xs = tuple(int(v) for v in rng.integers(0, V, n))
        p[xs] += rng.random() * 50
        p /= p.sum()
        m = T.marginals(p)
        if tuple(int(np.argmax(mj)) for mj in m) != xs:
            continue
        eps_j = np.array([1 - mj[xs[j]] for j, mj in enumerate(m)])
        if T.nonuniform_budget_ok(eps_j):
            hits += 1
            assert T.argmax_set(p) == [xs]
    assert hits > 100
