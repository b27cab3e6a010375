"""Pins of the oracle's binary64 gated delta update against facts the pages
and the algebra fix (not against a retyped copy of the update).

Pages: e-cogni STEPQuant analysis, "Como funciona" (Proposition 1: the error
carried by the update is scaled by the gate; the component along the current
key is further reduced by the write strength, orthogonal components are not)
and "Limitações" (its premise: identical inputs and gates); "Contexto" (GDN
scalar gate, KDA per-channel gate)."""
import numpy as np
import pytest


def _unit(rng, d):
    x = rng.standard_normal(d)
    return x / np.linalg.norm(x)


@pytest.mark.parametrize("seed", range(5))
def test_prop1_error_propagation_gdn(orc, seed):
    rng = np.random.default_rng(seed)
    dk, dv = 32, 24
    S = rng.standard_normal((dk, dv))
    E = 1e-3 * rng.standard_normal((dk, dv))
    q, k, v = _unit(rng, dk), _unit(rng, dk), rng.standard_normal(dv)
    k *= 1.3  # |k| != 1 on purpose: the factor is a(1 - b|k|^2)
    a, b = 0.93, 0.4
    S1, _ = orc.update_f64(S, q, k, v, a, b)
    S2, _ = orc.update_f64(S + E, q, k, v, a, b)
    dE = S2 - S1
    kk = k @ k
    khat = k / np.sqrt(kk)
    # along k: scaled by a (1 - b |k|^2)
    np.testing.assert_allclose(khat @ dE, a * (1 - b * kk) * (khat @ E), rtol=1e-9, atol=1e-13)
    # orthogonal to k: scaled by a only
    P = np.eye(dk) - np.outer(khat, khat)
    np.testing.assert_allclose(P @ dE, a * (P @ E), rtol=1e-9, atol=1e-13)


def test_prop1_kda_form(orc):
    rng = np.random.default_rng(7)
    dk, dv = 16, 8
    S, E = rng.standard_normal((dk, dv)), 1e-3 * rng.standard_normal((dk, dv))
    q, k, v = _unit(rng, dk), _unit(rng, dk), rng.standard_normal(dv)
    a = rng.uniform(0.5, 1.0, dk)
    b = 0.7
    dE = orc.update_f64(S + E, q, k, v, a, b)[0] - orc.update_f64(S, q, k, v, a, b)[0]
    expect = (np.eye(dk) - b * np.outer(k, k)) @ np.diag(a) @ E
    np.testing.assert_allclose(dE, expect, rtol=1e-9, atol=1e-14)


@pytest.mark.parametrize("seed", range(3))
def test_delta_rule_retrieval(orc, seed):
    """b = 1 and |k| = 1: the written value is read back exactly, S'^T k = v."""
    rng = np.random.default_rng(seed)
    S = rng.standard_normal((64, 48))
    k = _unit(rng, 64)
    v = rng.standard_normal(48)
    Sp, o = orc.update_f64(S, k, k, v, 0.97, 1.0)
    np.testing.assert_allclose(Sp.T @ k, v, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(o, v, rtol=1e-12, atol=1e-12)   # q = k reads v


def test_b0_is_pure_decay(orc):
    rng = np.random.default_rng(3)
    S = rng.standard_normal((16, 16))
    q, k, v = _unit(rng, 16), _unit(rng, 16), rng.standard_normal(16)
    Sp, o = orc.update_f64(S, q, k, v, 0.8, 0.0)
    np.testing.assert_array_equal(Sp, 0.8 * S)
    np.testing.assert_allclose(o, (0.8 * S).T @ q, rtol=1e-13)


def test_kda_constant_gate_equals_gdn(orc):
    rng = np.random.default_rng(4)
    S = rng.standard_normal((32, 32))
    q, k, v = _unit(rng, 32), _unit(rng, 32), rng.standard_normal(32)
    g1 = orc.update_f64(S, q, k, v, 0.9, 0.3)
    g2 = orc.update_f64(S, q, k, v, np.full(32, 0.9), 0.3)
    np.testing.assert_array_equal(g1[0], g2[0])
    np.testing.assert_array_equal(g1[1], g2[1])


@pytest.mark.parametrize("seed", range(4))
def test_bruteforce_4x4_product_form(orc, seed):
    """Tiny tiles: the oracle equals the closed product form
    S' = a (I - b k k^T) S + b k v^T and the readout S'^T q (GDN), and
    S' = (I - b k k^T) Diag(a) S + b k v^T (KDA)."""
    rng = np.random.default_rng(100 + seed)
    S = rng.standard_normal((4, 4))
    q, k, v = rng.standard_normal(4), rng.standard_normal(4), rng.standard_normal(4)
    a, b = rng.uniform(0.5, 1), rng.uniform(0, 1)
    Sp, o = orc.update_f64(S, q, k, v, a, b)
    ref = a * (np.eye(4) - b * np.outer(k, k)) @ S + b * np.outer(k, v)
    np.testing.assert_allclose(Sp, ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(o, ref.T @ q, rtol=1e-12, atol=1e-12)
    av = rng.uniform(0.5, 1, 4)
    Sp2, _ = orc.update_f64(S, q, k, v, av, b)
    ref2 = (np.eye(4) - b * np.outer(k, k)) @ np.diag(av) @ S + b * np.outer(k, v)
    np.testing.assert_allclose(Sp2, ref2, rtol=1e-12, atol=1e-12)


def test_fused_readout_form(orc):
    """o = S'^T q equals A^T q + delta (k.q) (the readout shares the update's pass)."""
    rng = np.random.default_rng(9)
    S = rng.standard_normal((64, 64))
    q, k, v = _unit(rng, 64), _unit(rng, 64), rng.standard_normal(64)
    a, b = 0.95, 0.6
    Sp, o = orc.update_f64(S, q, k, v, a, b)
    A = a * S
    delta = b * (v - A.T @ k)
    np.testing.assert_allclose(o, A.T @ q + delta * (k @ q), rtol=1e-11, atol=1e-12)
