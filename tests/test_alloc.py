"""The library's bit allocation (stq_allocate_bits, host code) against the
oracle (oracle/alloc.py): the same optimum as the 0/1 program on random
synthetic tables (per-unit error tables falling about 4x per extra bit with
heavy-tailed unit scales, GDN-like half-lives), pivots as the rule picks
them, the budget respected, host-side argument checks; above the size of
the exact table, the greedy path within one unit's gain of the linear
relaxation's optimum."""
import numpy as np
import pytest

from oracle import alloc


@pytest.fixture(scope="module")
def stq():
    import quantized_linear_attention_amd as q
    return q


def _tables(seed, n):
    g = np.random.default_rng(seed)
    sig = np.exp(g.normal(0, 1.5, n))
    err = sig[:, None] * 4.0 ** -np.array([4, 6, 8])[None, :] * g.uniform(0.5, 1.5, (n, 3))
    hl = np.clip(6.58 / g.uniform(0, 1, n), 6.58, 6931)
    return err, hl


@pytest.mark.parametrize("seed,n,n_piv,budget", [
    (1, 32, 1, 6.0), (2, 32, 0, 5.0), (3, 64, 2, 6.3), (4, 40, 0, 4.0), (5, 40, 3, 8.0),
    (6, 120, 4, 6.0), (7, 200, 0, 7.25), (8, 9, 2, 6.0)])
def test_exact_matches_oracle(stq, seed, n, n_piv, budget):
    err, hl = _tables(seed, n)
    bits, obj = stq.stq_allocate_bits(err, hl, n_piv, budget)
    ob, ov = alloc.allocate_milp(err, hl, n_piv, budget)
    assert abs(obj - ov) <= 1e-9 * max(1.0, ov)
    assert alloc.objective(err, hl, bits) == pytest.approx(obj, rel=1e-12)
    assert sorted(np.flatnonzero(bits == 16)) == alloc.pivots(err, hl, n_piv)
    q = bits[bits != 16]
    assert set(q) <= {4, 6, 8} and q.sum() <= budget * q.size + 1e-9


def test_small_matches_enumeration(stq):
    for seed in range(5):
        err, hl = _tables(100 + seed, 7)
        for n_piv, budget in [(0, 6.0), (1, 5.5), (2, 7.0)]:
            bits, obj = stq.stq_allocate_bits(err, hl, n_piv, budget)
            _, v = alloc.allocate_bruteforce(err, hl, n_piv, budget)
            assert abs(obj - v) <= 1e-12 * max(1.0, v)


def test_greedy_path_near_lp_optimum(stq):
    # m (K + 1) > 2^26 takes the greedy path: 9000 units at a 6-bit budget
    err, hl = _tables(9, 9000)
    bits, obj = stq.stq_allocate_bits(err, hl, 16, 6.0)
    lb = alloc.lp_bound(err, hl, 16, 6.0)
    w = alloc.lifetime_weight(hl)
    gap = float((w[:, None] * err).max(axis=1).max())
    assert lb <= obj + 1e-9 * obj and obj - lb <= gap
    q = bits[bits != 16]
    assert q.sum() <= 6.0 * q.size and (bits == 16).sum() == 16


def test_rejects_bad_arguments(stq):
    err, hl = _tables(0, 4)
    for args in [(err, hl, 5, 6.0), (err, hl, -1, 6.0), (err, hl, 0, 3.9), (err, -hl, 0, 6.0),
                 (-err, hl, 0, 6.0), (err, hl, 0, float("nan"))]:
        with pytest.raises(stq.StqError):
            stq.stq_allocate_bits(*args)
