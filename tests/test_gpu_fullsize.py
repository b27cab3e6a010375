"""GPU checks at the workloads' full launch sizes, against hand-derived values,
and a free-running report of how the quantized trajectories drift.

- The ingest (stq_pool_store) of the hand-derived refit examples (row-impact
  weights that differ per row, row factors that need bf16 rounding, reciprocal
  multiplies, exact-product code rounding), each embedded in a 128 x 128 tile:
  zero rows and columns change nothing else (zero rows have no exponent,
  zero columns scale 1), so the stored values must be the derivation's.
- The per-key-row KDA step at B = 256 and the windowed step at B = 512 over a
  whole window (16 tokens, the fold included), also with four compensator rows
  per tile: the launches the benchmark times, with sampled tiles re-stepped by
  the oracle from the GPU's bytes (teacher-forced), to the fused step's bar.
- The prefill at the benchmark's size (64 prompts of 1,024 tokens, P3, P4
  and P5), two sampled requests re-run by the oracle, to the prefill bars.
- Free-running over each decode configuration's own length (C3 64 tokens,
  C4 32, C5 64): the GPU pool and the oracle's pool each advance on their
  own from the same ingested state, next to the exact binary64 recurrence
  without any quantization.  Reported (per-step error
  feeding forward is what the pages quantify), gated only on finiteness.
"""
import numpy as np
import pytest

from gpu_util import Pair, add_agg, agg_text, compare_codes, new_agg, readout_ok, say
from test_gpu_parity import _assert_codes
from test_oracle_refit import REFIT_GOLDENS, load_refit_golden
from workloads import Workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available()
    return torch


def _bf16(bits):
    return (np.asarray(bits, np.uint32) << 16).view(np.float32).astype(np.float64)


def test_store_hand_derived_goldens(torch_cuda, orc):
    """Ingest on the GPU of the hand-derived refit examples, one per head."""
    from types import SimpleNamespace
    say("case ingest of hand-derived refit examples")
    gold = [load_refit_golden(g) for g in REFIT_GOLDENS]
    H, dk, dv = len(gold), 128, 128
    bits = np.array([int(g["n"][0]) for g in gold], np.int32)
    assert all(len(set(g["n"])) == 1 for g in gold)          # one width per example
    w = np.ones((H, dk), np.float32)
    S = np.zeros((1, H, dk, dv), np.float32)
    for h, g in enumerate(gold):
        Sg = np.array(g["S"], np.float32)
        S[0, h, :Sg.shape[0], :Sg.shape[1]] = Sg
        w[h, :Sg.shape[0]] = g["w"]
    wl = SimpleNamespace(B=1, H=H, dk=dk, dv=dv, cfg=SimpleNamespace(gate=0, unit=0, window=0), bits=bits,
                         row_weight=w)
    P = Pair(orc, wl, n_slots=1)
    P.store(np.array([0]), S)
    img = P.image()
    np.testing.assert_array_equal(img, P.ref.img)
    for h, g in enumerate(gold):
        Q, sg, cg, _ = P.ref.decode_tile(0, h, img)
        r, c = np.array(g["S"]).shape
        E = int(g["E"][0])
        np.testing.assert_array_equal(Q[:r, :c], np.array(g["Q"], np.int64), err_msg=REFIT_GOLDENS[h])
        assert not Q[r:].any() and not Q[:, c:].any()
        np.testing.assert_array_equal(_bf16(sg)[:r], g["sigma"])
        np.testing.assert_array_equal(_bf16(sg)[r:], 2.0 ** -E)          # zero rows: factor 1
        np.testing.assert_array_equal(_bf16(cg)[:c], g["c"])
        np.testing.assert_array_equal(_bf16(cg)[c:], 2.0 ** E)           # zero columns: scale 1


def test_full_c4_step_sampled(torch_cuda, orc):
    """KDA per-channel gate, per-key-row widths, B = 256 (the benchmark's
    launch): one step over every slot, 16 sampled slots (512 tiles) re-stepped
    by the oracle from the GPU's bytes."""
    say("case full C4 sampled")
    wl = Workload("C4")
    P = Pair(orc, wl)
    slots = np.arange(wl.B)
    P.store(slots, wl.state(slots))
    r_all = new_agg()
    rng = np.random.default_rng(41)
    for t in range(2):
        pre = P.image()
        q, k, v, a, b = wl.token(t)
        o = P.gpu_step(slots, q, k, v, a, b)
        post = P.image()
        samp = np.sort(rng.choice(wl.B, 16, replace=False))
        ref = orc.OraclePool(wl.B, wl.H, wl.dk, wl.dv, np.asarray(wl.bits).reshape(-1), wl.row_weight,
                             wl.cfg.gate, wl.cfg.unit, 0, image=pre)
        o_ref = ref.step(samp, q[samp], k[samp], v[samp], a[samp], b[samp])
        add_agg(r_all, compare_codes(orc, ref, post, ref.img, samp), readout_ok(o[samp], o_ref))
        assert np.isfinite(o).all()
    say("  full C4: %s, readout %.3f" % (agg_text(r_all), r_all["o"]))
    _assert_codes(r_all)
    assert r_all["o"] <= 1.0


def test_full_c5_window_sampled(torch_cuda, orc):
    """Windowed 4-bit pool, B = 512, W = 16 (the benchmark's launches): a whole
    window of 16 tokens, the fold included.  At every token 16 sampled slots
    are re-stepped by the oracle from the GPU's bytes: readout, cached Gamma
    and k bit-exact, cached u within 1e-4; the base unchanged inside the
    window; at the fold the new base's codes to the fused step's bar."""
    say("case full C5 window sampled")
    wl = Workload("C5")
    W = wl.cfg.window
    P = Pair(orc, wl)
    slots = np.arange(wl.B)
    P.store(slots, wl.state(slots))
    rng = np.random.default_rng(51)
    agg = new_agg()
    worst_o = worst_u = 0.0
    for t in range(W):
        pre = P.image()
        q, k, v, a, b = wl.token(t)
        o = P.gpu_step(slots, q, k, v, a, b)
        post = P.image()
        samp = np.sort(rng.choice(wl.B, 16, replace=False))
        ref = orc.OraclePool(wl.B, wl.H, wl.dk, wl.dv, wl.bits, wl.row_weight, window=W, image=pre)
        o_ref = ref.step(samp, q[samp], k[samp], v[samp], a[samp], b[samp])
        worst_o = max(worst_o, readout_ok(o[samp], o_ref))
        for s in samp[:4]:
            for h in range(wl.H):
                cg, Gg, Kg, Ug, _, _ = ref.cache_view(int(s), h, post)
                cr, Gr, Kr, Ur, _, _ = ref.cache_view(int(s), h)
                assert cg == cr == (t + 1) % W
                np.testing.assert_array_equal(Gg[:cg], Gr[:cr])
                np.testing.assert_array_equal(Kg[:cg], Kr[:cr])
                if cg:
                    worst_u = max(worst_u, float(np.abs(Ug[:cg] - Ur[:cr]).max() / np.abs(Ur[:cr]).max()))
        if t + 1 == W:
            add_agg(agg, compare_codes(orc, ref, post, ref.img, samp))
        else:
            for s in samp[:4]:
                for h in range(wl.H):
                    np.testing.assert_array_equal(ref.tile_view(int(s), h, post), ref.tile_view(int(s), h, pre))
        assert np.isfinite(o).all()
    say("  full C5: readout %.3f, cache u %.2e, fold: %s" % (worst_o, worst_u, agg_text(agg)))
    assert worst_o <= 1.0
    assert worst_u <= 1e-4
    _assert_codes(agg)


def test_full_c5_compensators_sampled(torch_cuda, orc):
    """The windowed 4-bit pool at B = 512, W = 16, with four compensator rows
    per tile (the pages' outlier terms riding the window's update path): a
    whole window, the fold included, with 16 sampled slots re-stepped by the
    oracle from the GPU's bytes at every token: readout, cached Gamma and k
    bit-exact, cached u within 1e-4, the kept rows' indices exact and values
    within 1e-5 relative; at the fold the new base's codes to the fused
    step's bar."""
    say("case full C5 with compensators sampled")
    wl = Workload("C5")
    W, C = wl.cfg.window, 4
    P = Pair(orc, wl, n_comp=C)
    slots = np.arange(wl.B)
    P.store(slots, wl.state(slots))
    rng = np.random.default_rng(53)
    agg = new_agg()
    worst_o = worst_u = worst_c = 0.0
    for t in range(W):
        pre = P.image()
        q, k, v, a, b = wl.token(t)
        o = P.gpu_step(slots, q, k, v, a, b)
        post = P.image()
        samp = np.sort(rng.choice(wl.B, 16, replace=False))
        ref = orc.OraclePool(wl.B, wl.H, wl.dk, wl.dv, wl.bits, wl.row_weight, window=W, image=pre, n_comp=C)
        o_ref = ref.step(samp, q[samp], k[samp], v[samp], a[samp], b[samp])
        worst_o = max(worst_o, readout_ok(o[samp], o_ref))
        for s in samp[:4]:
            for h in range(wl.H):
                cg, Gg, Kg, Ug, ig, vg = ref.cache_view(int(s), h, post)
                cr, Gr, Kr, Ur, ir, vr = ref.cache_view(int(s), h)
                assert cg == cr == (t + 1) % W
                np.testing.assert_array_equal(Gg[:cg], Gr[:cr])
                np.testing.assert_array_equal(Kg[:cg], Kr[:cr])
                if cg:
                    worst_u = max(worst_u, float(np.abs(Ug[:cg] - Ur[:cr]).max() / np.abs(Ur[:cr]).max()))
                np.testing.assert_array_equal(ig, ir)
                if (ir >= 0).any():
                    worst_c = max(worst_c, float(np.abs(vg - vr).max() / np.abs(vr).max()))
        if t + 1 == W:
            add_agg(agg, compare_codes(orc, ref, post, ref.img, samp))
        assert np.isfinite(o).all()
    say("  full C5 C=4: readout %.3f, cache u %.2e, compensators %.2e, fold: %s"
        % (worst_o, worst_u, worst_c, agg_text(agg)))
    assert worst_o <= 1.0
    assert worst_u <= 1e-4
    assert worst_c <= 1e-5
    _assert_codes(agg)


def _exact_step(S, q, k, v, a, b):
    """The gated delta rule in binary64 on unquantized states [n][H][dk][dv]:
    A = a S (scalar gate per (request, head)) or Diag(a) S (per-channel gate,
    a [n][H][dk]), S' = A + k (b (v - A^T k))^T, o = S'^T q."""
    S = S * (a[..., :, None] if a.ndim == 3 else a[..., None, None])
    u = np.einsum("nhij,nhi->nhj", S, k)
    S = S + k[..., :, None] * (b[..., None] * (v - u))[..., None, :]
    return S, np.einsum("nhij,nhi->nhj", S, q)


# the configurations' own lengths: C3 64 tokens, C4 32, C5 64 (four windows)
FREE_RUNS = [("C3", 64), ("C4", 32), ("C5", 64)]


@pytest.mark.parametrize("key,T", FREE_RUNS)
def test_free_running_report(torch_cuda, orc, key, T):
    """Each configuration's generator over its own length, 16 requests x 32
    heads: the GPU pool and the oracle's pool step on their own (no teacher
    forcing).  Reported per token: the GPU's and the oracle's readout error
    against the exact unquantized recurrence (from the same decoded start),
    the GPU-vs-oracle readout difference and the fraction of codes in which
    the two pools differ (window pools: the base, rewritten at each fold)."""
    say("case free-running %s, %d tokens" % (key, T))
    wl = Workload(key, B=16)
    P = Pair(orc, wl)
    slots = np.arange(wl.B)
    P.store(slots, wl.state(slots))
    S = P.ref.fetch(slots).astype(np.float64)
    rel = lambda x, y: float(np.abs(x - y).max() / np.abs(y).max())
    say("  token  gpu-vs-exact  oracle-vs-exact  gpu-vs-oracle  codes differing")
    for t in range(T):
        q, k, v, a, b = wl.token(t)
        o_g = P.gpu_step(slots, q, k, v, a, b).astype(np.float64)
        o_r = P.ref.step(slots, q, k, v, a, b)
        S, o_x = _exact_step(S, q.astype(np.float64), k.astype(np.float64), v.astype(np.float64),
                             a.astype(np.float64), b.astype(np.float64))
        assert np.isfinite(o_g).all()
        if t + 1 in (1, 2, 4, 8, 16, 32, 64):
            r = compare_codes(orc, P.ref, P.image(), P.ref.img, slots)
            say("  %5d  %12.2e  %15.2e  %13.2e  %15.2e"
                % (t + 1, rel(o_g, o_x), rel(o_r, o_x), rel(o_g, o_r), r["mism"] / max(r["codes"], 1)))


@pytest.mark.parametrize("key", ["P3", "P4", "P5"])
def test_full_prefill_sampled(torch_cuda, orc, key):
    """The prefill at the size the benchmark times (bench.py's own setup: 64
    prompts of 1,024 tokens in one stq_prefill call; P3 into the C3 pool with
    GDN gates, P4 the same head mix with per-channel gates, P5 into the
    per-key-row C4 pool with per-channel gates).  Two
    sampled requests (all 32 heads) are re-run by the oracle from the pool's
    bytes before the call: every readout of their 2,048 tokens, their final
    states and their codes, to the prefill bars of test_gpu_prefill."""
    import bench
    from test_gpu_prefill import _assert_prefill_codes, _state_ok
    torch = torch_cuda
    B, Lp = 64, 1024
    say("case full-size prefill", key, B, Lp)
    st = bench.prefill_setup(key, B, Lp, torch.device("cuda:0"))
    wl = st["wl"]
    torch.cuda.synchronize()
    pre = st["buf"].cpu().numpy()
    import quantized_linear_attention_amd as stq
    stq.stq_prefill(st["pool"], st["slots"], st["ss"], st["q"], st["k"], st["v"], st["a"], st["b"], st["o"])
    torch.cuda.synchronize()
    img = st["buf"].cpu().numpy()
    sample = np.array([0, 37], np.int32)                         # slot c holds prompt c
    tok = torch.as_tensor(np.concatenate([np.arange(c * Lp, (c + 1) * Lp) for c in sample]), device="cuda")
    host = {x: st[x][tok].cpu().numpy() for x in "qkvab"}      # the sampled prompts' tokens only
    o = st["o"][tok].cpu().numpy()
    c = wl.cfg
    ref = orc.OraclePool(B, wl.H, wl.dk, wl.dv, np.asarray(wl.bits).reshape(-1), wl.row_weight, c.gate, c.unit, 0,
                         image=pre)
    ss = np.arange(0, len(sample) * Lp + 1, Lp, dtype=np.int32)
    o_ref, S_fin = ref.prefill(sample, ss, host["q"], host["k"], host["v"], host["a"], host["b"], final_state=True)
    T = len(tok)
    r = readout_ok(o.reshape(T, 1, wl.H, wl.dv), o_ref.reshape(T, 1, wl.H, wl.dv))
    w = _state_ok(orc, ref, img, sample, S_fin, [True] * len(sample))
    res = compare_codes(orc, ref, img, ref.img, sample)
    say("  %s: readout worst ratio %.3g, state worst ratio %.3g, %s" % (key, r, w, agg_text(res)))
    assert r <= 1.0
    assert w <= 1.0
    _assert_prefill_codes(res)
