"""Pins of the per-key-row bit allocation (KDA, unit = key row: gpt-diffusion
STEPQuant analysis, "Las dos ideas") in the oracle: hand-derived row-record
bytes, round trips at every width mix, and pool behaviour (pivot rows kept in
binary16 outside the row/column fits)."""
import os

import numpy as np
import pytest

from workloads import Workload

GOLD = os.path.join(os.path.dirname(__file__), "golden", "row_records.txt")


def test_row_record_golden(orc):
    rows, widths, expect = {}, None, None
    for line in open(GOLD):
        if line.startswith("#") or not line.strip():
            continue
        key, *rest = line.split()
        if key == "widths":
            widths = np.array([int(x) for x in rest], np.int32)
        elif key == "row":
            rows[int(rest[0])] = [int(x) for x in rest[1:]]
        elif key == "bytes":
            off = int(rest[0])
            expect = (off, np.array([int(x, 16) for x in rest[1:]], np.uint8))
    Q = np.array([rows[i] for i in range(4)], np.int32)
    one = np.full(4, 0x3F80, np.uint16)
    t = orc.pack_rows(widths, Q, one, np.full(8, 0x3F80, np.uint16))
    assert t.size == 54
    off, b = expect
    np.testing.assert_array_equal(t[off:off + b.size], b)
    np.testing.assert_array_equal(t[30:38].view(np.uint16), one)


@pytest.mark.parametrize("seed", range(4))
def test_row_roundtrip(orc, seed):
    rng = np.random.default_rng(seed)
    dk, dv = 128, 128
    nb = rng.choice([4, 6, 8, 16], dk, p=[0.3, 0.5, 0.19, 0.01]).astype(np.int32)
    Q = np.zeros((dk, dv), np.int32)
    for i in range(dk):
        if nb[i] == 16:
            Q[i] = rng.integers(0, 0x7C00, dv)
        else:
            qm = 2 ** (nb[i] - 1) - 1
            Q[i] = rng.integers(-qm, qm + 1, dv)
    sig = rng.integers(0, 1 << 16, dk).astype(np.uint16)
    c = rng.integers(0, 1 << 16, dv).astype(np.uint16)
    t = orc.pack_rows(nb, Q, sig, c)
    assert t.size == sum(dv * n // 8 for n in nb) + 2 * (dk + dv)
    Q2, s2, c2 = orc.unpack_rows(nb, dv, t)
    np.testing.assert_array_equal(Q2, Q)
    np.testing.assert_array_equal(s2, sig)
    np.testing.assert_array_equal(c2, c)


def test_kda_pool_store_step(orc):
    wl = Workload("C4", B=3, H=4)
    P = orc.OraclePool(4, wl.H, wl.dk, wl.dv, wl.bits.reshape(-1), wl.row_weight, gate_kind=1, unit_kind=1)
    slots = np.array([3, 0, 2])
    S0 = wl.state(slots)
    P.store(slots, S0)
    assert np.all(P.fetch([1]) == 0)
    for c, s in enumerate(slots):
        for h in range(wl.H):
            nb = wl.bits[h]
            sig, cs, Q, _ = orc.refit(S0[c, h], wl.row_weight[h], nb)
            np.testing.assert_array_equal(P.tile_view(s, h), orc.pack_rows(nb, Q, sig, cs))
            piv = nb == 16
            D = P.fetch([s])[0, h]
            # pivot rows are the binary16 of the state, outside the fits
            np.testing.assert_array_equal(D[piv], np.clip(S0[c, h][piv], -65504, 65504).astype(np.float16).astype(np.float32))
    Shat = P.fetch(slots)
    q, k, v, a, b = wl.token(0, 3)
    o = P.step(slots, q, k, v, a, b)
    for c, s in enumerate(slots):
        for h in range(wl.H):
            Sp, oref = orc.update_f64(Shat[c, h], q[c, h], k[c, h], v[c, h], a[c, h], b[c, h])
            np.testing.assert_allclose(o[c, h], oref, rtol=1e-13, atol=1e-13)
            sig, cs, Q, _ = orc.refit(Sp.astype(np.float32), wl.row_weight[h], wl.bits[h])
            np.testing.assert_array_equal(P.tile_view(s, h), orc.pack_rows(wl.bits[h], Q, sig, cs))
    assert orc.clip_events() == 0
