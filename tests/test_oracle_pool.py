"""Pool-level oracle behaviour: pool image = per-tile encodings at the
documented offsets; the step = R of the binary64 update; the identity rule;
the fixed-scale round trip."""
import numpy as np
import pytest

from workloads import Workload


def _pool(orc, wl, n_slots, window=0):
    return orc.OraclePool(n_slots, wl.H, wl.dk, wl.dv, wl.bits, wl.row_weight,
                          gate_kind=wl.cfg.gate, window=window)


def test_fresh_pool_is_zero_state(orc):
    wl = Workload("C2", B=3, H=4)
    P = _pool(orc, wl, 5)
    S = P.fetch(np.arange(5))
    assert np.all(S == 0)
    hdr = P.img[:64].view(np.uint32)
    assert hdr[0] == 0x31515453 and hdr[1] == 5 and hdr[2] == 4


def test_store_fetch_matches_tile_functions(orc):
    wl = Workload("C2", B=3, H=6)
    P = _pool(orc, wl, 7)
    slots = np.array([5, 0, 3])
    S0 = wl.state(slots)
    P.store(slots, S0)
    back = P.fetch(slots)
    for c, s in enumerate(slots):
        for h in range(wl.H):
            n = int(wl.bits[h])
            sig, cs, Q, _ = orc.refit(S0[c, h], wl.row_weight[h], n)
            np.testing.assert_array_equal(P.tile_view(s, h), orc.pack(n, Q, sig, cs))
            np.testing.assert_array_equal(back[c, h], orc.dequant(sig, cs, Q, n))
    # untouched slots stay zero
    assert np.all(P.fetch([1, 2, 4, 6]) == 0)


@pytest.mark.parametrize("key", ["C1", "C2"])
def test_step_is_refit_of_f64_update(orc, key):
    wl = Workload(key, B=3, H=min(4, Workload(key).H))
    P = _pool(orc, wl, 4)
    slots = np.array([2, 0, 3])
    P.store(slots, wl.state(slots))
    Shat = P.fetch(slots)
    q, k, v, a, b = wl.token(0, 3)
    o = P.step(slots, q, k, v, a, b)
    for c, s in enumerate(slots):
        for h in range(wl.H):
            Sp, oref = orc.update_f64(Shat[c, h], q[c, h], k[c, h], v[c, h], a[c, h], b[c, h])
            np.testing.assert_allclose(o[c, h], oref, rtol=1e-13, atol=1e-13)
            n = int(wl.bits[h])
            sig, cs, Q, _ = orc.refit(Sp.astype(np.float32), wl.row_weight[h], n)
            np.testing.assert_array_equal(P.tile_view(s, h), orc.pack(n, Q, sig, cs))


def test_identity_update_keeps_bytes(orc):
    """b = 0 and a = 1: the codes (every byte) are unchanged and o = S^T q."""
    wl = Workload("C2", B=4, H=8)
    P = _pool(orc, wl, 4)
    slots = np.arange(4)
    P.store(slots, wl.state(slots))
    before = P.img.copy()
    Shat = P.fetch(slots)
    q, k, v, a, b = wl.token(0, 4)
    o = P.step(slots, q, k, v, np.ones_like(a), np.zeros_like(b))
    np.testing.assert_array_equal(P.img, before)
    ref = np.einsum("chij,chi->chj", Shat.astype(np.float64), q.astype(np.float64))
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)
    # KDA gate vector of ones
    wk = Workload("C1", B=2)
    Pk = orc.OraclePool(2, wk.H, wk.dk, wk.dv, wk.bits, wk.row_weight, gate_kind=1)
    Pk.store([0, 1], wk.state([0, 1]))
    bk = Pk.img.copy()
    Pk.step([0, 1], *wk.token(0, 2)[:3], np.ones((2, wk.H, wk.dk), np.float32), np.zeros((2, wk.H)))
    np.testing.assert_array_equal(Pk.img, bk)


def test_fixed_scale_requant_keeps_bytes(orc):
    wl = Workload("C2", B=4, H=8)
    P = _pool(orc, wl, 4)
    slots = np.arange(4)
    P.store(slots, wl.state(slots))
    for t in range(2):
        P.step(slots, *wl.token(t, 4))
    before = P.img.copy()
    P.requant_fixed(slots)
    np.testing.assert_array_equal(P.img, before)
