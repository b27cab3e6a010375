"""Pins of the oracle's refit R (encoding) and dequantisation D.

Pages: STEPQuant talk preview (qingkeai.online), "STEPQuant 核心设计…"
(separate key-row and value-column scales, row scale from the row's current
magnitude and its impact); e-cogni analysis, "Como funciona" (square-root
smoothing, geometric-mean normalisation); gpt-diffusion analysis, "Qué dice
realmente el «6-bit»" (16-bit scales).  Checks use closed forms derived by
hand (tests/golden), exact symmetries of the definition, a textbook special
case, and brute-force enumeration of codes."""
import os

import numpy as np
import pytest

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def bf16(bits):
    return (np.asarray(bits, np.uint32) << 16).view(np.float32)


def test_rank1_closed_form(orc):
    vals = {}
    Qrows = []
    for line in open(os.path.join(GOLD, "refit_rank1_8bit.txt")):
        if line.startswith("#") or not line.strip():
            continue
        key, *rest = line.split()
        if key == "Q":
            Qrows.append([int(x) for x in rest])
        else:
            vals[key] = [float(x) for x in rest]
    x = np.array([1, 4, 16, 64.0])
    y = np.array([1, -4, 2, -16.0])
    sig, c, Q, E = orc.refit(np.outer(x, y), np.ones(4), 8)
    assert E == int(vals["E"][0])
    np.testing.assert_array_equal(bf16(sig), np.array(vals["sigma"], np.float32))
    np.testing.assert_array_equal(bf16(c), np.array(vals["c"], np.float32))
    np.testing.assert_array_equal(Q, np.array(Qrows))
    assert orc.clip_events() == 0


def load_refit_golden(name):
    """A hand-derived refit example: rows of S, row weights w, row widths n,
    and the expected E, stored sigma and c (as values) and codes Q."""
    g = {"S": [], "Q": []}
    for line in open(os.path.join(GOLD, name)):
        if line.startswith("#") or not line.strip():
            continue
        key, *rest = line.split()
        if key in ("S", "Q"):
            g[key].append([float(x) for x in rest])
        else:
            g[key] = [float(x) for x in rest]
    return g


REFIT_GOLDENS = ["refit_impact_weight_8bit.txt", "refit_row_factor_rne_8bit.txt",
                 "refit_reciprocals_4bit.txt"]


def check_refit_golden(refit, name):
    """Run `refit` (oracle.refit's signature) on the golden's input; return the
    list of outputs that differ from the hand derivation."""
    g = load_refit_golden(name)
    S = np.array(g["S"], np.float32)
    w = np.array(g["w"], np.float32)
    nb = np.array(g["n"], np.int32)
    # the inputs are exact binary32 values
    assert np.array_equal(S.astype(np.float64), np.array(g["S"])) and np.array_equal(w.astype(np.float64), g["w"])
    sig, c, Q, E = refit(S, w, nb)
    bad = []
    if E != int(g["E"][0]):
        bad.append("E")
    if not np.array_equal(bf16(sig).astype(np.float64), g["sigma"]):
        bad.append("sigma")
    if not np.array_equal(bf16(c).astype(np.float64), g["c"]):
        bad.append("c")
    if not np.array_equal(Q, np.array(g["Q"], np.int64)):
        bad.append("Q")
    return bad


@pytest.mark.parametrize("name", REFIT_GOLDENS)
def test_refit_hand_derived(orc, name):
    """Row-impact weights that differ per row, row factors that need bf16
    round-to-nearest-even, and the reciprocal multiplies and exact-product
    rounding of the column fit and the codes, each against a hand derivation."""
    assert check_refit_golden(orc.refit, name) == []
    assert orc.clip_events() == 0


def _rand_tile(rng, dk, dv, spread=1.5):
    r = np.exp(rng.normal(0, spread, dk))
    c = np.exp(rng.normal(0, spread, dv))
    return (rng.standard_normal((dk, dv)) * r[:, None] * c[None, :]).astype(np.float32)


@pytest.mark.parametrize("n", [4, 6, 8])
def test_equivariances(orc, n):
    rng = np.random.default_rng(n)
    dk, dv = 16, 12
    S = _rand_tile(rng, dk, dv)
    w = np.exp(rng.normal(0, 1, dk)).astype(np.float32)
    sig, c, Q, E = orc.refit(S, w, n)
    # row permutation (weights permuted with the rows)
    p = rng.permutation(dk)
    s2, c2, Q2, _ = orc.refit(S[p], w[p], n)
    np.testing.assert_array_equal(s2, sig[p]); np.testing.assert_array_equal(c2, c)
    np.testing.assert_array_equal(Q2, Q[p])
    # column permutation
    pc = rng.permutation(dv)
    s3, c3, Q3, _ = orc.refit(S[:, pc], w, n)
    np.testing.assert_array_equal(s3, sig); np.testing.assert_array_equal(c3, c[pc])
    np.testing.assert_array_equal(Q3, Q[:, pc])
    # sign flip
    s4, c4, Q4, _ = orc.refit(-S, w, n)
    np.testing.assert_array_equal(s4, sig); np.testing.assert_array_equal(c4, c)
    np.testing.assert_array_equal(Q4, -Q)
    # S -> 4^k S: codes and row scales unchanged, column scales times 4^k
    for kexp in (-3, 1, 2):
        s5, c5, Q5, E5 = orc.refit(S * np.float32(4.0 ** kexp), w, n)
        np.testing.assert_array_equal(Q5, Q)
        np.testing.assert_array_equal(s5, sig)
        np.testing.assert_array_equal(bf16(c5), bf16(c) * np.float32(4.0 ** kexp))
        assert E5 == E + kexp
    # w -> 4^k w: nothing stored changes (normalisation absorbs it)
    s6, c6, Q6, _ = orc.refit(S, w * np.float32(16.0), n)
    np.testing.assert_array_equal(s6, sig); np.testing.assert_array_equal(c6, c)
    np.testing.assert_array_equal(Q6, Q)
    assert orc.clip_events() == 0


def _bf16_ceil(x):
    """Smallest bfloat16 >= x > 0 (8 significant bits), by np.frexp."""
    m, e = np.frexp(np.asarray(x, np.float64))     # x = m 2^e, m in [0.5, 1)
    return np.ceil(m * 256.0) / 256.0 * np.exp2(e)


@pytest.mark.parametrize("n", [4, 6, 8])
def test_textbook_per_column_absmax(orc, n):
    """When every row has the same m_i w_i (here 4^j times a common power of
    four) the row factors are all one power of two and R reduces to symmetric
    per-column absmax quantisation with the step rounded up to bf16."""
    rng = np.random.default_rng(20 + n)
    dk, dv = 8, 10
    S = rng.uniform(-1, 1, (dk, dv)).astype(np.float32)
    S[:, 0] = 1.0                                   # every row absmax = 1
    w = np.full(dk, 4.0, np.float32)                 # m w = 4 -> factor 2 for all rows
    sig, c, Q, E = orc.refit(S, w, n)
    qmax = 2 ** (n - 1) - 1
    step = _bf16_ceil(np.abs(S).max(axis=0).astype(np.float64) * np.float64(np.float32(1.0 / qmax)))
    # stored sigma*c equals the per-column step
    np.testing.assert_array_equal((bf16(sig)[:, None] * bf16(c)[None, :]).astype(np.float64),
                                  np.broadcast_to(step, (dk, dv)))
    expect = np.rint(S.astype(np.float64) / step)
    np.testing.assert_array_equal(Q, expect)


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("n", [4, 6, 8])
def test_bruteforce_nearest_code_4x4(orc, seed, n):
    """Enumerate every code: the chosen one is the nearest grid point to S
    with the fitted scales, no code is clipped, and the grid covers each
    column (its largest code is qmax or qmax - 1)."""
    rng = np.random.default_rng(1000 * n + seed)
    S = _rand_tile(rng, 4, 4, 1.0)
    w = rng.uniform(0.5, 2, 4).astype(np.float32)
    sig, c, Q, E = orc.refit(S, w, n)
    qmax = 2 ** (n - 1) - 1
    step = bf16(sig)[:, None].astype(np.float64) * bf16(c)[None, :]
    codes = np.arange(-qmax, qmax + 1)
    err = np.abs(S[..., None].astype(np.float64) - step[..., None] * codes)
    best = err.min(axis=-1)
    chosen = np.abs(S - step * Q)
    assert np.all(chosen <= best * (1 + 1e-6) + 1e-30)
    assert np.all(np.abs(Q) <= qmax)
    assert np.all(np.abs(Q).max(axis=0) >= qmax - 1)
    assert orc.clip_events() == 0


def test_zero_and_degenerate_tiles(orc):
    # all-zero tile: codes 0, scales 1
    sig, c, Q, E = orc.refit(np.zeros((8, 8), np.float32), np.ones(8), 6)
    assert E == 0 and np.all(Q == 0)
    assert np.all(bf16(sig) == 1) and np.all(bf16(c) == 1)
    # a zero row and a zero column: scale 1 for the row (times 2^-E), codes 0
    rng = np.random.default_rng(5)
    S = rng.standard_normal((8, 8)).astype(np.float32)
    S[3] = 0; S[:, 5] = 0
    sig, c, Q, E = orc.refit(S, np.ones(8), 8)
    assert np.all(Q[3] == 0) and np.all(Q[:, 5] == 0)
    assert bf16(sig)[3] == np.float32(2.0 ** -E)
    assert bf16(c)[5] == np.float32(2.0 ** E)
    # single non-zero element
    S = np.zeros((8, 8), np.float32); S[2, 6] = -3.5
    sig, c, Q, E = orc.refit(S, np.ones(8), 4)
    assert Q[2, 6] in (-7, -6) and np.count_nonzero(Q) == 1


def test_pivot_rows_binary16(orc):
    rng = np.random.default_rng(6)
    S = _rand_tile(rng, 8, 8)
    S[0, 0] = 1e6            # saturates to 65504 in a pivot row
    nb = np.array([16, 6, 6, 6, 6, 6, 6, 16])
    sig, c, Q, E = orc.refit(S, np.ones(8), nb)
    for i in (0, 7):
        got = Q[i].astype(np.uint16).view(np.float16).astype(np.float32)
        ref = np.clip(S[i], -65504, 65504).astype(np.float16).astype(np.float32)
        np.testing.assert_array_equal(got, ref)
    # pivot rows do not influence the column scales
    S2 = S.copy(); S2[0] *= 100; S2[7] *= 0.01
    sig2, c2, Q2, _ = orc.refit(S2, np.ones(8), nb)
    np.testing.assert_array_equal(c2, c)
    np.testing.assert_array_equal(Q2[1:7], Q[1:7])


@pytest.mark.parametrize("n", [4, 6, 8])
def test_dequant_exact_and_fixed_scale_roundtrip(orc, n):
    """D is exact (checked in binary64) and Q_{sigma,c}(D(Q)) = Q for every
    code at random scales: quantize/dequantize round-trip idempotence."""
    rng = np.random.default_rng(30 + n)
    qmax = 2 ** (n - 1) - 1
    dk, dv = 16, 2 * qmax + 1
    Q = np.tile(np.arange(-qmax, qmax + 1), (dk, 1)).astype(np.int32)   # every code
    sig = (rng.uniform(0.01, 50, dk).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    c = (rng.uniform(1e-4, 2, dv).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    S = orc.dequant(sig, c, Q, n)
    exact = bf16(sig).astype(np.float64)[:, None] * bf16(c).astype(np.float64)[None, :] * Q
    np.testing.assert_array_equal(S.astype(np.float64), exact)
    np.testing.assert_array_equal(orc.requant_fixed(S, sig, c, n), Q)


@pytest.mark.parametrize("n", [4, 6, 8])
def test_refit_of_decode_drift_is_small(orc, n):
    """R(D(R(S))) is not a projection (the row factor follows the decoded row
    absmax); measure how many codes move and by how much."""
    rng = np.random.default_rng(40 + n)
    S = _rand_tile(rng, 128, 128)
    w = np.exp(rng.normal(0, 1.15, 128)).astype(np.float32)
    sig, c, Q, _ = orc.refit(S, w, n)
    sig2, c2, Q2, _ = orc.refit(orc.dequant(sig, c, Q, n), w, n)
    moved = np.mean(Q2 != Q)
    print("R(D(R(S))) drift n=%d: %.4f of codes moved, max |dQ| %d"
          % (n, moved, np.abs(Q2 - Q).max()))
    assert moved < 0.25


def test_refit_of_decoded_tile_is_not_idempotent(orc):
    """Why no exact 'refit of a decoded tile keeps its codes' invariant exists
    under these readings, even holding the row scales: the column scale is
    rounded UP to bf16 from the column's absmax, and a decoded column's absmax
    sits below the one it was fitted to.  Worked by hand on a 1 x 1, 8-bit tile:
      S = 1: s = 1, E = 0; M = fl(1/127) = 8454660 * 2^-30 -> t = 130 * 2^-14,
        Q = rne(1 * fl(16384/130)) = rne(126.03) = 126;
      D: fl(130 * 2^-14) * 126 = 16380 * 2^-14 = 4095/4096;
      refit of 4095/4096: s = bf16(sqrt(4095/4096)) = bf16(0.99988) = 1 (same row
        scale), M = fl(4095/4096 * fl(1/127)) = 2^-7 * 1.00763 -> t' = 129 * 2^-14,
        Q' = rne(4095/4096 * fl(16384/129)) = rne(126.98) = 127.
    The row scale is unchanged, yet c and Q both move.  The exact invariant that
    does hold, requantizing against the stored scales, is checked in
    test_dequant_exact_and_fixed_scale_roundtrip."""
    sig, c, Q, E = orc.refit(np.array([[1.0]], np.float32), np.ones(1, np.float32), 8)
    assert E == 0 and bf16(sig)[0] == 1.0 and bf16(c)[0] == 130 * 2.0 ** -14 and Q[0, 0] == 126
    D = orc.dequant(sig, c, Q, 8)
    assert D[0, 0] == np.float32(4095 / 4096)
    sig2, c2, Q2, E2 = orc.refit(D, np.ones(1, np.float32), 8)
    assert E2 == 0 and bf16(sig2)[0] == 1.0                       # row scale held
    assert bf16(c2)[0] == 129 * 2.0 ** -14 and Q2[0, 0] == 127     # column scale and code moved
