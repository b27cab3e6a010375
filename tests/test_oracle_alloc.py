"""Pins of the oracle's lifetime-aware bit allocation (oracle/alloc.py).

  - the lifetime weight: closed form of the geometric series at h = 1 (= 2),
    against a long explicit sum, and its large-h asymptote h / ln 2 + 1/2;
  - a two-unit example worked by hand;
  - exhaustive enumeration and the MILP formulation agree on random instances;
  - the budget extremes: 4 bits gives every unit 4, 8 bits gives every unit 8;
  - the pivots are the units of largest lifetime-weighted 8-bit error.
"""
import math

import numpy as np
import pytest

from oracle import alloc


def test_lifetime_weight():
    assert alloc.lifetime_weight(1.0) == 2.0
    h = 3.7
    s = sum(2.0 ** (-t / h) for t in range(4000))
    assert abs(alloc.lifetime_weight(h) - s) <= 1e-12 * s
    for h in (1e3, 1e5):
        assert abs(alloc.lifetime_weight(h) - (h / math.log(2) + 0.5)) <= 1e-3


def test_two_units_by_hand():
    # equal lifetimes; budget 6 bits on average: (8, 4) costs 1 + 5 = 6, (6, 6) 4 + 3 = 7, (4, 8) 12.5
    err = np.array([[10.0, 4.0, 1.0], [5.0, 3.0, 2.5]])
    hl = np.array([1.0, 1.0])
    bits, v = alloc.allocate_bruteforce(err, hl, 0, 6.0)
    assert list(bits) == [8, 4] and v == 2.0 * 6.0
    bits, v = alloc.allocate_milp(err, hl, 0, 6.0)
    assert list(bits) == [8, 4] and abs(v - 12.0) < 1e-9


@pytest.mark.parametrize("seed", range(6))
def test_bruteforce_equals_milp(seed):
    g = np.random.default_rng(seed)
    n = 7
    sig = np.exp(g.normal(0, 1, n))
    err = sig[:, None] * 4.0 ** -np.array([4, 6, 8])[None, :] * g.uniform(0.5, 1.5, (n, 3))
    hl = np.clip(6.58 / g.uniform(0, 1, n), 6.58, 6931)
    for n_piv, budget in [(0, 6.0), (1, 5.3), (2, 7.1), (0, 4.0), (1, 8.0)]:
        b1, v1 = alloc.allocate_bruteforce(err, hl, n_piv, budget)
        b2, v2 = alloc.allocate_milp(err, hl, n_piv, budget)
        assert abs(v1 - v2) <= 1e-9 * max(1.0, abs(v1))
        assert alloc.objective(err, hl, b2) == pytest.approx(v2, rel=1e-12)
        q = b2[b2 != 16]
        assert q.sum() <= budget * q.size + 1e-9
        assert lb_ok(err, hl, n_piv, budget, v1)


def lb_ok(err, hl, n_piv, budget, v):
    return alloc.lp_bound(err, hl, n_piv, budget) <= v + 1e-9 * max(1.0, v)


def test_budget_extremes_and_pivots():
    g = np.random.default_rng(11)
    n = 6
    err = np.sort(g.uniform(0.1, 1.0, (n, 3)), axis=1)[:, ::-1].copy()
    hl = g.uniform(5, 500, n)
    b, _ = alloc.allocate_bruteforce(err, hl, 0, 4.0)
    assert set(b) == {4}
    b, _ = alloc.allocate_bruteforce(err, hl, 0, 8.0)
    assert set(b) == {8}
    risk = alloc.lifetime_weight(hl) * err[:, 2]
    b, _ = alloc.allocate_bruteforce(err, hl, 2, 6.0)
    assert sorted(np.flatnonzero(b == 16)) == sorted(np.argsort(-risk)[:2])
