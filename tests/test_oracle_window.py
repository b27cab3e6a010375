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
