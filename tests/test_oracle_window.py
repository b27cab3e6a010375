"""Window mode of the oracle (LeapQuant post, technique one: the low-bit
state is frozen inside a token window, per-token updates are cached at high
precision and the readout uses both; requantize at the window end)."""
import numpy as np

from workloads import Workload


def _setup(orc, W, slots=3, H=2):
    wl = Workload("C5", B=slots, H=H)
    P = orc.OraclePool(slots, H, wl.dk, wl.dv, wl.bits, wl.row_weight, window=W)
    sl = np.arange(slots)
    P.store(sl, wl.state(sl))
    return wl, P, sl


def _recurrence(S0, toks, c, h):
    """Per-token recurrence from S0 with binary32 cache semantics: gates are
    the ratios of the binary32 running products, written vectors rounded to
    binary32."""
    S = S0.astype(np.float64)
    G_prev = None
    outs = []
    for (q, k, v, a, b) in toks:
        G = np.float32(a[c, h]) if G_prev is None else np.float32(G_prev * np.float32(a[c, h]))
        g = float(G) if G_prev is None else float(G) / float(G_prev)
        G_prev = G
        kk = k[c, h].astype(np.float64)
        u = (b[c, h] * (v[c, h] - g * S.T @ kk)).astype(np.float32).astype(np.float64)
        S = g * S + np.outer(kk, u)
        outs.append(S.T @ q[c, h].astype(np.float64))
    return S, outs


def test_window_readout_equals_recurrence(orc):
    W = 16
    wl, P, sl = _setup(orc, W)
    S0 = P.fetch(sl)
    toks = [wl.token(t, sl.size) for t in range(10)]
    outs = [P.step(sl, *tk) for tk in toks]
    for c in sl:
        for h in range(wl.H):
            _, ref = _recurrence(S0[c, h], toks, c, h)
            for t in range(10):
                np.testing.assert_allclose(outs[t][c, h], ref[t], rtol=1e-9, atol=1e-9)
    # the base is frozen inside the window
    np.testing.assert_array_equal(P.fetch(sl), S0)


def test_window_fold_is_refit_of_materialized_state(orc):
    W = 4
    wl, P, sl = _setup(orc, W)
    S0 = P.fetch(sl)
    toks = [wl.token(t, sl.size) for t in range(W)]
    for tk in toks:
        P.step(sl, *tk)
    for c in sl:
        for h in range(wl.H):
            SW, _ = _recurrence(S0[c, h], toks, c, h)
            sig, cs, Q, _ = orc.refit(SW.astype(np.float32), wl.row_weight[h], int(wl.bits[h]))
            np.testing.assert_array_equal(P.tile_view(c, h), orc.pack(int(wl.bits[h]), Q, sig, cs))


def test_flush_empty_window_is_noop_and_flush_folds(orc):
    wl, P, sl = _setup(orc, 16)
    before = P.img.copy()
    P.window_flush(sl)
    np.testing.assert_array_equal(P.img, before)
    S0 = P.fetch(sl)
    toks = [wl.token(t, sl.size) for t in range(3)]
    for tk in toks:
        P.step(sl, *tk)
    P.window_flush(sl)
    for c in sl:
        for h in range(wl.H):
            S3, _ = _recurrence(S0[c, h], toks, c, h)
            sig, cs, Q, _ = orc.refit(S3.astype(np.float32), wl.row_weight[h], int(wl.bits[h]))
            np.testing.assert_array_equal(P.tile_view(c, h), orc.pack(int(wl.bits[h]), Q, sig, cs))
    # the window restarted: next readout uses the new base only
    S1 = P.fetch(sl)
    q, k, v, a, b = wl.token(9, sl.size)
    o = P.step(sl, q, k, v, a, b)
    _, ref = _recurrence(S1[0, 0], [(q, k, v, a, b)], 0, 0)
    np.testing.assert_allclose(o[0, 0], ref[0], rtol=1e-9, atol=1e-9)


# ---- compensator tokens (LeapQuant post, technique two) ----

def _top_rows(S, C):
    """Rows taken as compensators, written independently of the oracle: order
    by row absmax, largest first, ties to the lower row, zero rows never."""
    m = np.abs(S.astype(np.float32)).max(axis=1)
    order = np.lexsort((np.arange(S.shape[0]), -m.astype(np.float64)))
    rows = [int(i) for i in order[:C] if m[i] > 0]
    return rows + [-1] * (C - len(rows))


def _residual(S, rows):
    R = S.astype(np.float32).copy()
    for i in rows:
        if i >= 0:
            R[i] = 0.0
    return R


def _planted(wl, sl, seed=3):
    rng = np.random.default_rng(seed)
    S = wl.state(sl).copy()
    for c in range(S.shape[0]):
        for h in range(S.shape[1]):
            for r, f in zip(rng.choice(wl.dk, 3, replace=False), (60.0, 40.0, 25.0)):
                S[c, h, r] *= f
    return S


def test_compensators_take_the_largest_rows_exactly(orc):
    W, C = 8, 4
    wl = Workload("C5", B=3, H=2)
    sl = np.arange(3)
    S = _planted(wl, sl)
    P = orc.OraclePool(3, 2, wl.dk, wl.dv, wl.bits, wl.row_weight, window=W, n_comp=C)
    P.store(sl, S)
    F = P.fetch(sl)
    for c in sl:
        for h in range(2):
            rows = _top_rows(S[c, h], C)
            cnt, _, _, _, idx, val = P.cache_view(c, h)
            assert cnt == 0
            np.testing.assert_array_equal(idx, rows)
            for k, i in enumerate(rows):
                np.testing.assert_array_equal(val[k], S[c, h, i])        # kept exactly
                np.testing.assert_array_equal(F[c, h, i], S[c, h, i])
            # the base is R of the residual
            sig, cs, Q, _ = orc.refit(_residual(S[c, h], rows), wl.row_weight[h], int(wl.bits[h]))
            np.testing.assert_array_equal(P.tile_view(c, h), orc.pack(int(wl.bits[h]), Q, sig, cs))


def test_compensators_lower_the_error_of_the_other_rows(orc):
    wl = Workload("C5", B=2, H=2)
    sl = np.arange(2)
    S = _planted(wl, sl, seed=5)
    err = {}
    for C in (0, 3):
        P = orc.OraclePool(2, 2, wl.dk, wl.dv, wl.bits, wl.row_weight, window=8, n_comp=C)
        P.store(sl, S)
        e = np.abs(P.fetch(sl) - S)
        err[C] = e.max(axis=3).mean()
    assert err[3] < 0.5 * err[0]


def test_compensator_ties_zero_rows_and_pivot_heads(orc):
    dk = dv = 64
    bits = np.array([4, 16], np.int32)
    wt = np.ones((2, dk), np.float32)
    S = np.zeros((1, 2, dk, dv), np.float32)
    S[0, :, 9, 3] = 2.0
    S[0, :, 4, 7] = -2.0          # same absmax: the lower row first
    S[0, :, 30, 0] = 0.5
    P = orc.OraclePool(1, 2, dk, dv, bits, wt, window=4, n_comp=5)
    P.store(np.arange(1), S)
    _, _, _, _, idx, _ = P.cache_view(0, 0)
    np.testing.assert_array_equal(idx, [4, 9, 30, -1, -1])
    _, _, _, _, idx, val = P.cache_view(0, 1)    # a binary16 pivot head takes none
    np.testing.assert_array_equal(idx, [-1] * 5)
    assert not val.any()
    np.testing.assert_array_equal(P.fetch(np.arange(1)), S)


def test_compensated_window_readout_equals_recurrence(orc):
    W, C = 8, 3
    wl = Workload("C5", B=3, H=2)
    sl = np.arange(3)
    P = orc.OraclePool(3, 2, wl.dk, wl.dv, wl.bits, wl.row_weight, window=W, n_comp=C)
    P.store(sl, _planted(wl, sl))
    S0 = P.fetch(sl)                               # base plus compensators
    toks = [wl.token(t, sl.size) for t in range(W - 1)]
    outs = [P.step(sl, *tk) for tk in toks]
    for c in sl:
        for h in range(2):
            _, ref = _recurrence(S0[c, h], toks, c, h)
            for t in range(W - 1):
                np.testing.assert_allclose(outs[t][c, h], ref[t], rtol=1e-9, atol=1e-9)


def test_compensated_fold_extracts_then_refits(orc):
    W, C = 4, 3
    wl = Workload("C5", B=2, H=2)
    sl = np.arange(2)
    P = orc.OraclePool(2, 2, wl.dk, wl.dv, wl.bits, wl.row_weight, window=W, n_comp=C)
    P.store(sl, _planted(wl, sl, seed=7))
    S0 = P.fetch(sl)
    toks = [wl.token(t, sl.size) for t in range(W)]
    for tk in toks:
        P.step(sl, *tk)
    for c in sl:
        for h in range(2):
            SW, _ = _recurrence(S0[c, h], toks, c, h)
            SW = SW.astype(np.float32)
            rows = _top_rows(SW, C)
            cnt, _, _, _, idx, val = P.cache_view(c, h)
            assert cnt == 0
            np.testing.assert_array_equal(idx, rows)
            for k, i in enumerate(rows):
                np.testing.assert_array_equal(val[k], SW[i])
            sig, cs, Q, _ = orc.refit(_residual(SW, rows), wl.row_weight[h], int(wl.bits[h]))
            np.testing.assert_array_equal(P.tile_view(c, h), orc.pack(int(wl.bits[h]), Q, sig, cs))
