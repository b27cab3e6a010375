"""Pins of the oracle's prefill ingest against closed forms and other code paths.

The prefill runs the per-token gated delta rule in binary64 from D(tile) and
writes R(fl32(S_T)) once (LeapQuant post, section on decode cost and state
memory under prefix caching).  Pins:
  - the chunkwise form of the same recurrence, written independently here with
    a dense linear solve (no sequential scan): final state and every readout;
  - b = 0: pure decay, S_T = (prod a) S_0 and o_t = (prod_{r<=t} a_r) S_0^T q_t;
  - delta-rule retrieval: a = 1, b = 1, orthonormal keys: S_T^T k_s = v_s;
  - one token = the oracle's decode step (bytes and readout), GDN and KDA;
  - no tokens / identity tokens leave the tile; the written tile is the
    oracle's own store of fl32(S_T); requests are independent of each other;
  - window pools: with an empty window and no compensators, exactly the plain
    pool's prefill; otherwise the prompt starts from the folded state with its
    compensators (checked by pure decay) and ends as the ingest's store;
  - per-channel gates: each row decays by its own gates (b = 0), and one token
    is the decode step.
"""
import numpy as np
import pytest

import oracle
from workloads import Workload


def _pool(wl, n_slots, seed=0):
    c = wl.cfg
    P = oracle.OraclePool(n_slots, wl.H, wl.dk, wl.dv, wl.bits, wl.row_weight, c.gate, c.unit, 0)
    P.store(np.arange(n_slots), wl.state(np.arange(n_slots) + 100 * seed))
    return P


def _chunk_form(S0, q, k, v, a, b):
    """Final state and readouts of one (request, head) by the chunkwise form:
    gamma_t = prod_{r<=t} a_r, ratio[t, s] = prod_{s<r<=t} a_r (products, no
    division), (I + A) Delta = diag(b) (V - diag(gamma) K S0) with
    A[t, s] = b_t ratio[t, s] k_t.k_s (s < t); S_T = gamma_T S0 + K^T diag(ratio[T-1, :]) Delta;
    O = diag(gamma) Q S0 + (tril(ratio * Q K^T)) Delta."""
    T = q.shape[0]
    a = a.astype(np.float64)
    b = b.astype(np.float64)
    K, Q, V = k.astype(np.float64), q.astype(np.float64), v.astype(np.float64)
    gam = np.cumprod(a)
    ratio = np.zeros((T, T))
    for t in range(T):
        for s in range(t + 1):
            ratio[t, s] = np.prod(a[s + 1:t + 1])
    A = np.tril(b[:, None] * ratio * (K @ K.T), -1)
    rhs = b[:, None] * (V - gam[:, None] * (K @ S0))
    Delta = np.linalg.solve(np.eye(T) + A, rhs)
    ST = gam[-1] * S0 + K.T @ (ratio[-1][:, None] * Delta)
    O = gam[:, None] * (Q @ S0) + np.tril(ratio * (Q @ K.T)) @ Delta
    return ST, O


def test_chunk_form_matches_recurrence():
    wl = Workload("C1")
    P = _pool(wl, 3)
    S0 = P.fetch(np.arange(3)).astype(np.float64)
    lens = [37, 1, 20]
    ss, q, k, v, a, b = wl.prompts(lens)
    o, Sf = P.prefill(np.arange(3), ss, q, k, v, a, b, final_state=True)
    for c in range(3):
        t0, t1 = ss[c], ss[c + 1]
        for h in range(wl.H):
            ST, O = _chunk_form(S0[c, h], q[t0:t1, h], k[t0:t1, h], v[t0:t1, h], a[t0:t1, h], b[t0:t1, h])
            sc = np.abs(ST).max()
            assert np.abs(Sf[c, h] - ST).max() <= 1e-11 * sc
            assert np.abs(o[t0:t1, h] - O).max() <= 1e-11 * max(1.0, np.abs(O).max())


def test_pure_decay():
    wl = Workload("C1")
    P = _pool(wl, 2)
    S0 = P.fetch(np.arange(2)).astype(np.float64)
    ss, q, k, v, a, b = wl.prompts([9, 4])
    b[:] = 0
    o, Sf = P.prefill(np.arange(2), ss, q, k, v, a, b, final_state=True)
    for c in range(2):
        t0, t1 = ss[c], ss[c + 1]
        for h in range(wl.H):
            ah = a[t0:t1, h].astype(np.float64)
            assert np.allclose(Sf[c, h], np.prod(ah) * S0[c, h], rtol=1e-13, atol=0)
            for t in range(t1 - t0):
                want = np.prod(ah[:t + 1]) * (S0[c, h].T @ q[t0 + t, h].astype(np.float64))
                assert np.allclose(o[t0 + t, h], want, rtol=1e-12, atol=1e-14)


def test_delta_rule_retrieval():
    """a = 1, b = 1, orthonormal keys: each written value is read back exactly,
    whatever the initial state (the write replaces the state's old value along k)."""
    wl = Workload("C1")
    P = _pool(wl, 1)
    T = 24
    g = np.random.default_rng(7)
    ss = np.array([0, T], np.int32)
    k = np.zeros((T, wl.H, wl.dk), np.float32)
    for h in range(wl.H):
        Qm, _ = np.linalg.qr(g.standard_normal((wl.dk, wl.dk)))
        k[:, h] = Qm[:, :T].T
    v = g.standard_normal((T, wl.H, wl.dv)).astype(np.float32)
    q = k.copy()                                   # read token t's own key
    a = np.ones((T, wl.H), np.float32)
    b = np.ones((T, wl.H), np.float32)
    o, Sf = P.prefill([0], ss, q, k, v, a, b, final_state=True)
    kd = k.astype(np.float64)
    # k is binary32-rounded: orthonormal to ~1e-7, so retrieval holds to that level
    for h in range(wl.H):
        for s in range(T):
            assert np.allclose(Sf[0, h].T @ kd[s, h], v[s, h], atol=1e-5)
            assert np.allclose(o[s, h], v[s, h], atol=1e-5)


@pytest.mark.parametrize("key", ["C1", "C2", "C4"])
def test_one_token_is_a_decode_step(key):
    wl = Workload(key, B=3, H=4)
    c = wl.cfg
    P1 = oracle.OraclePool(3, wl.H, wl.dk, wl.dv, wl.bits, wl.row_weight, c.gate, c.unit, 0)
    P1.store(np.arange(3), wl.state(np.arange(3)))
    P2 = oracle.OraclePool(3, wl.H, wl.dk, wl.dv, wl.bits, wl.row_weight, c.gate, c.unit, 0, image=P1.img)
    q, k, v, a, b = wl.token(0, n=3)
    o1 = P1.step([2, 0, 1], q, k, v, a, b)
    ss = np.arange(4, dtype=np.int32)
    o2 = P2.prefill([2, 0, 1], ss, q, k, v, a, b)
    assert np.array_equal(P1.img, P2.img)
    assert np.array_equal(o1, o2)


def test_identity_and_empty_leave_the_tile():
    wl = Workload("C2", B=3, H=4)
    P = _pool(wl, 3)
    before = P.img.copy()
    ss, q, k, v, a, b = wl.prompts([0, 5, 0])
    a[:] = 1.0
    b[:] = 0.0
    P.prefill(np.arange(3), ss, q, k, v, a, b)
    assert np.array_equal(P.img, before)
    # one non-identity token anywhere in a request rewrites that request only
    b[3, :] = 0.5
    P.prefill(np.arange(3), ss, q, k, v, a, b)
    for s in range(3):
        for h in range(wl.H):
            same = np.array_equal(P.tile_view(s, h), oracle.OraclePool(
                3, wl.H, wl.dk, wl.dv, wl.bits, wl.row_weight, 0, 0, 0, image=before).tile_view(s, h))
            assert same == (s != 1)


def test_written_tile_is_store_of_final_state():
    wl = Workload("C2", B=2, H=6)
    P = _pool(wl, 4)
    Q = oracle.OraclePool(4, wl.H, wl.dk, wl.dv, wl.bits, wl.row_weight, 0, 0, 0, image=P.img)
    ss, q, k, v, a, b = wl.prompts([13, 40])
    o, Sf = P.prefill([3, 1], ss, q, k, v, a, b, final_state=True)
    Q.store([3, 1], Sf.astype(np.float32))
    assert np.array_equal(P.img, Q.img)


def test_requests_are_independent():
    wl = Workload("C1")
    P = _pool(wl, 3)
    Q = oracle.OraclePool(3, wl.H, wl.dk, wl.dv, wl.bits, wl.row_weight, 0, 0, 0, image=P.img)
    ss, q, k, v, a, b = wl.prompts([7, 0, 19])
    o = P.prefill([0, 1, 2], ss, q, k, v, a, b)
    for c in (2, 0):                                  # one request per call, other order
        t0, t1 = ss[c], ss[c + 1]
        oc = Q.prefill([c], np.array([0, t1 - t0], np.int32), q[t0:t1], k[t0:t1], v[t0:t1], a[t0:t1], b[t0:t1])
        assert np.array_equal(oc, o[t0:t1])
    assert np.array_equal(P.img, Q.img)


def _window_pool(wl, n_slots, W, C):
    P = oracle.OraclePool(n_slots, wl.H, wl.dk, wl.dv, wl.bits, wl.row_weight, 0, 0, W, n_comp=C)
    P.store(np.arange(n_slots), wl.state(np.arange(n_slots)))
    return P


def test_window_pool_empty_window_is_plain_prefill():
    """No compensators and an empty window: the same tiles and readouts as a pool without a window."""
    wl = Workload("C5", B=2, H=4)
    Pw = _window_pool(wl, 2, 16, 0)
    Pp = oracle.OraclePool(2, wl.H, wl.dk, wl.dv, wl.bits, wl.row_weight, 0, 0, 0)
    Pp.store(np.arange(2), wl.state(np.arange(2)))
    ss, q, k, v, a, b = wl.prompts([21, 40])
    ow = Pw.prefill([0, 1], ss, q, k, v, a, b)
    op = Pp.prefill([0, 1], ss, q, k, v, a, b)
    assert np.array_equal(ow, op)
    for s in range(2):
        for h in range(wl.H):
            assert np.array_equal(Pw.tile_view(s, h), Pp.tile_view(s, h))


def test_window_pool_starts_from_folded_state_with_compensators():
    """Pure decay (b = 0, a = 1/2): the final state is 2^-T times the state the
    pool holds after its open window is folded, compensators included; the
    written base and compensators are the store of that final state."""
    wl = Workload("C5", B=2, H=4)
    P = _window_pool(wl, 2, 8, 3)
    q0, k0, v0, a0, b0 = wl.token(0, n=2)
    P.step([0, 1], q0, k0, v0, a0, b0)                     # open a window of one token
    F = oracle.OraclePool(2, wl.H, wl.dk, wl.dv, wl.bits, wl.row_weight, 0, 0, 8, image=P.img, n_comp=3)
    F.window_flush([0, 1])
    S_folded = F.fetch([0, 1]).astype(np.float64)
    ss, q, k, v, a, b = wl.prompts([5, 9])
    a[:] = 0.5
    b[:] = 0.0
    o, Sf = P.prefill([0, 1], ss, q, k, v, a, b, final_state=True)
    for c, T in enumerate([5, 9]):
        assert np.array_equal(Sf[c], S_folded[c] * 0.5 ** T)
    F.store([0, 1], Sf.astype(np.float32))
    assert np.array_equal(P.img, F.img)


def _kda_head_pool(n_slots):
    import dataclasses
    wl = Workload("C4", B=n_slots, H=4)
    wl.cfg = dataclasses.replace(wl.cfg, unit=0)
    wl.bits = np.array([4, 6, 8, 16], np.int32)
    P = oracle.OraclePool(n_slots, wl.H, wl.dk, wl.dv, wl.bits, wl.row_weight, 1, 0, 0)
    P.store(np.arange(n_slots), wl.state(np.arange(n_slots)))
    return wl, P


def test_per_channel_pure_decay():
    """Per-channel gates, b = 0: row i decays by the product of its own gates."""
    wl, P = _kda_head_pool(2)
    S0 = P.fetch(np.arange(2)).astype(np.float64)
    ss, q, k, v, a, b = wl.prompts([6, 3])
    b[:] = 0
    o, Sf = P.prefill([0, 1], ss, q, k, v, a, b, final_state=True)
    for c in range(2):
        t0, t1 = ss[c], ss[c + 1]
        for h in range(wl.H):
            ah = a[t0:t1, h].astype(np.float64)                 # [T][dk]
            assert np.allclose(Sf[c, h], np.prod(ah, axis=0)[:, None] * S0[c, h], rtol=1e-13, atol=0)
            for t in range(t1 - t0):
                g = np.prod(ah[:t + 1], axis=0)
                want = (g[:, None] * S0[c, h]).T @ q[t0 + t, h].astype(np.float64)
                assert np.allclose(o[t0 + t, h], want, rtol=1e-12, atol=1e-14)


def test_per_channel_one_token_is_a_decode_step():
    wl, P1 = _kda_head_pool(3)
    P2 = oracle.OraclePool(3, wl.H, wl.dk, wl.dv, wl.bits, wl.row_weight, 1, 0, 0, image=P1.img)
    q, k, v, a, b = wl.token(0, n=3)
    o1 = P1.step([1, 2, 0], q, k, v, a, b)
    o2 = P2.prefill([1, 2, 0], np.arange(4, dtype=np.int32), q, k, v, a, b)
    assert np.array_equal(P1.img, P2.img) and np.array_equal(o1, o2)
