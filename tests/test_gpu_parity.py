"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Bar (written here): store/fetch/fixed-scale requantization bit-exact; fused
step: code mismatch rate <= 1e-4 with every mismatch <= 1 code step, readout
within 1e-3 relative (per element, with a floor of 1% of the tile's largest
output), checked teacher-forced (the oracle steps from the GPU's bytes)."""
import numpy as np
import pytest

from gpu_util import Pair, add_agg, agg_text, compare_codes, new_agg, readout_ok, say
from workloads import Workload

pytestmark = pytest.mark.gpu

MISMATCH_MAX = 1e-4

# (config, B, slot-pool size, slot permutation seed): ragged request counts
STORE_CASES = [("C1", 4, 4), ("C2", 64, 64), ("C3", 37, 50), ("C4", 19, 23), ("C5", 21, 24)]


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available()
    return torch


@pytest.mark.parametrize("key,B,NS", STORE_CASES)
def test_create_and_store_bitexact(torch_cuda, orc, key, B, NS):
    say("case store", key, B, NS)
    wl = Workload(key, B=B)
    P = Pair(orc, wl, n_slots=NS)
    np.testing.assert_array_equal(P.image(), P.ref.img)          # header + zero state
    slots = np.random.default_rng(1).permutation(NS)[:B]
    P.store(slots, wl.state(slots))
    g = P.image()
    diff = np.nonzero(g != P.ref.img)[0]
    assert diff.size == 0, "first differing bytes at %s" % diff[:10]


@pytest.mark.parametrize("key,B,NS", STORE_CASES)
def test_fetch_and_fixed_requant_exact(torch_cuda, orc, key, B, NS):
    say("case fetch", key, B, NS)
    torch = torch_cuda
    wl = Workload(key, B=B)
    P = Pair(orc, wl, n_slots=NS)
    slots = np.arange(NS)[::-1][:B].copy()
    P.store(slots, wl.state(slots))
    out = torch.empty((B, wl.H, wl.dk, wl.dv), dtype=torch.float32, device="cuda")
    P.stq.stq_pool_fetch(P.pool, P.slots_t(slots), out)
    np.testing.assert_array_equal(out.cpu().numpy(), P.ref.fetch(slots))
    before = P.image()
    P.stq.stq_requant_fixed_scales(P.pool, P.slots_t(slots))
    np.testing.assert_array_equal(P.image(), before)


@pytest.mark.parametrize("key", ["C1", "C2", "C4"])
def test_identity_update_keeps_bytes(torch_cuda, orc, key):
    say("case identity", key)
    wl = Workload(key, B=min(16, Workload(key).B))
    P = Pair(orc, wl)
    slots = np.arange(wl.B)
    P.store(slots, wl.state(slots))
    before = P.image()
    q, k, v, a, b = wl.token(0)
    o = P.gpu_step(slots, q, k, v, np.ones_like(a), np.zeros_like(b))
    np.testing.assert_array_equal(P.image(), before)
    o_ref = P.ref.step(slots, q, k, v, np.ones_like(a), np.zeros_like(b))
    assert readout_ok(o, o_ref) <= 1.0


def _assert_codes(r):
    """Stored codes = integer codes of the quantized units + binary16 values of
    the pivot units.  Bar: combined mismatch <= 1e-4, integer codes <= 1e-4,
    every mismatch one step (one code, or one binary16 rounding).  A binary16
    grid is ~2^11 levels per binade, so binary32-vs-binary64 arithmetic alone
    flips ~1e-4 of pivot values by one ulp: those are bounded at 1e-3.
    Scales: the row and column scales (compared as the steps they define)
    differ in at most 1e-4 of them, each by one bf16 step."""
    assert (r["mism"] + r["piv_mism"]) <= MISMATCH_MAX * max(r["codes"] + r["piv"], 1)
    assert r["mism"] <= MISMATCH_MAX * max(r["codes"], 1)
    assert r["maxd"] <= 1
    assert r["piv_mism"] <= 1e-3 * max(r["piv"], 1)
    assert r["piv_bad"] == 0
    assert r["scale_mism"] <= MISMATCH_MAX * max(r["scales"], 1)
    assert r["scale_steps"] <= 1


def _teacher_forced(orc, wl, P, slots, T):
    worst = new_agg()
    for t in range(T):
        img = P.image()
        ref = orc.OraclePool(P.n_slots, wl.H, wl.dk, wl.dv, np.asarray(wl.bits).reshape(-1),
                             wl.row_weight, wl.cfg.gate, wl.cfg.unit, wl.cfg.window, image=img)
        q, k, v, a, b = wl.token(t, len(slots))
        o = P.gpu_step(slots, q, k, v, a, b)
        o_ref = ref.step(slots, q, k, v, a, b)
        r = compare_codes(orc, ref, P.image(), ref.img, slots)
        add_agg(worst, r, readout_ok(o, o_ref))
    return worst


@pytest.mark.parametrize("key,B,T", [("C1", 4, 32), ("C2", 64, 1), ("C3", 40, 4), ("C4", 24, 4)])
def test_fused_step_teacher_forced(torch_cuda, orc, key, B, T):
    say("case step", key, B, T)
    wl = Workload(key, B=B)
    P = Pair(orc, wl, n_slots=B + 3)
    slots = np.random.default_rng(2).permutation(B + 3)[:B]
    P.store(slots, wl.state(slots))
    r = _teacher_forced(orc, wl, P, slots, T)
    rate = r["mism"] / max(r["codes"], 1)
    say("  code mismatch %.2e (%d of %d), max |dQ| %d, scale mismatch %d of %d, pivot mismatch %d "
        "(beyond one step: %d) of %d, readout err/bound %.3f"
        % (rate, r["mism"], r["codes"], r["maxd"], r["scale_mism"], r["scales"], r["piv_mism"],
           r["piv_bad"], r["piv"], r["o"]))
    _assert_codes(r)
    assert r["o"] <= 1.0


def test_full_c3_step_sampled(torch_cuda, orc):
    """B = 512, H = 32, d = 128 (the benchmark shape, same launch): one step,
    512 sampled tiles re-stepped by the oracle from the GPU's bytes."""
    say("case full C3 sampled")
    wl = Workload("C3")
    P = Pair(orc, wl)
    slots = np.arange(512)
    P.store(slots, wl.state(slots))
    pre = P.image()
    q, k, v, a, b = wl.token(0)
    o = P.gpu_step(slots, q, k, v, a, b)
    post = P.image()
    rng = np.random.default_rng(11)
    samp = rng.choice(512, 16, replace=False)
    ref = orc.OraclePool(512, wl.H, wl.dk, wl.dv, wl.bits, wl.row_weight, image=pre)
    o_ref = ref.step(samp, q[samp], k[samp], v[samp], a[samp], b[samp])
    r = compare_codes(orc, ref, post, ref.img, samp)
    rate = r["mism"] / r["codes"]
    say("  sampled code mismatch %.2e, max |dQ| %d, pivot mismatch %d of %d, readout %.3f"
        % (rate, r["maxd"], r["piv_mism"], r["piv"], readout_ok(o[samp], o_ref)))
    _assert_codes(r)
    assert readout_ok(o[samp], o_ref) <= 1.0
    # untouched-by-sample tiles still decode to finite values
    assert np.isfinite(o).all()


@pytest.mark.parametrize("dk,dv", [(64, 128), (128, 64)])
def test_other_tile_shapes(torch_cuda, orc, dk, dv):
    say("case shape", dk, dv)
    wl = Workload("C2", B=6, H=8)
    wl.dk, wl.dv = dk, dv
    wl.row_weight = wl.row_weight[:, :dk].copy()
    rng = np.random.default_rng(dk + dv)
    wl.bits = np.array([4, 6, 8, 16, 6, 4, 8, 6], np.int32)
    P = Pair(orc, wl)
    slots = np.arange(6)
    S = (rng.standard_normal((6, 8, dk, dv)) * np.exp(rng.normal(0, 1.5, (1, 8, dk, 1)))).astype(np.float32)
    P.store(slots, S)
    np.testing.assert_array_equal(P.image(), P.ref.img)
    q = rng.standard_normal((6, 8, dk)); q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.standard_normal((6, 8, dk)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((6, 8, dv))
    a = rng.uniform(0.9, 1, (6, 8)); b = rng.uniform(0, 1, (6, 8))
    f = lambda x: x.astype(np.float32)
    pre = P.image()
    o = P.gpu_step(slots, f(q), f(k), f(v), f(a), f(b))
    ref = P.orc.OraclePool(6, 8, dk, dv, wl.bits, wl.row_weight, image=pre)
    o_ref = ref.step(slots, f(q), f(k), f(v), f(a), f(b))
    r = compare_codes(orc, ref, P.image(), ref.img, slots)
    say("  shape %dx%d: %s, readout %.3f" % (dk, dv, agg_text(r), readout_ok(o, o_ref)))
    _assert_codes(r)
    assert readout_ok(o, o_ref) <= 1.0


def _row_width_patterns(dk, rng):
    """Per-head key-row widths (original row order) that reach every path of the
    per-key-row step: one width only, binary16 pivots only, runs of a width that
    end inside a step of the kernel, a lone quantized row among pivots, a mix in
    the C4 proportions and a uniform random mix."""
    from workloads import quotas
    pats = [np.full(dk, 4), np.full(dk, 6), np.full(dk, 8), np.full(dk, 16),
            np.repeat([4, 6, 8, 16], [3, 5, dk - 9, 1]),
            np.repeat([4, 6, 8, 16], quotas([0.30, 0.50, 0.19, 0.01], dk)),
            np.repeat([8, 16], [1, dk - 1]),
            rng.choice([4, 6, 8, 16], dk)]
    return np.stack([rng.permutation(p) for p in pats]).astype(np.int32)


@pytest.mark.parametrize("dk,dv,gate", [(128, 128, 1), (64, 64, 1), (64, 128, 1), (128, 64, 1),
                                         (128, 128, 0), (64, 128, 0)])
def test_rows_step_shapes(torch_cuda, orc, dk, dv, gate):
    """Per-key-row widths at every tile shape, with the per-channel gate and
    (d_v = 128) the per-head gate: two teacher-forced steps (the oracle steps
    from the GPU's bytes each time)."""
    from types import SimpleNamespace
    say("case rows step", dk, dv, "gate", gate)
    rng = np.random.default_rng(100 + dk + dv + 7 * gate)
    H, B = 8, 6
    cfg = SimpleNamespace(gate=gate, unit=1, window=0)
    wl = SimpleNamespace(B=B, H=H, dk=dk, dv=dv, cfg=cfg, bits=_row_width_patterns(dk, rng),
                         row_weight=np.clip(np.exp(rng.normal(0, 1.15, (H, dk))), 0.1, 10).astype(np.float32))
    P = Pair(orc, wl, n_slots=B + 2)
    slots = rng.permutation(B + 2)[:B]
    prof = np.exp(rng.normal(0, 1.5, (1, H, dk, 1))) * np.exp(rng.normal(0, 1.5, (1, H, 1, dv)))
    P.store(slots, (0.1 * rng.standard_normal((B, H, dk, dv)) * prof).astype(np.float32))
    f = lambda x: x.astype(np.float32)
    worst = new_agg()
    for t in range(2):
        img = P.image()
        ref = orc.OraclePool(B + 2, H, dk, dv, wl.bits.reshape(-1), wl.row_weight, gate, 1, 0, image=img)
        q = rng.standard_normal((B, H, dk)); q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k = rng.standard_normal((B, H, dk)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
        v = rng.standard_normal((B, H, dv))
        a = 2.0 ** (-1.0 / (10.0 ** rng.uniform(0, 4, (B, H, dk) if gate else (B, H))))
        b = rng.uniform(0.05, 0.95, (B, H))
        o = P.gpu_step(slots, f(q), f(k), f(v), f(a), f(b))
        o_ref = ref.step(slots, f(q), f(k), f(v), f(a), f(b))
        r = compare_codes(orc, ref, P.image(), ref.img, slots)
        add_agg(worst, r, readout_ok(o, o_ref))
    say("  rows %dx%d gate %d: code mismatch %d of %d (max |dQ| %d), scale mismatch %d of %d, pivot mismatch %d of %d, "
        "readout %.3f" % (dk, dv, gate, worst["mism"], worst["codes"], worst["maxd"], worst["scale_mism"],
                          worst["scales"], worst["piv_mism"], worst["piv"], worst["o"]))
    _assert_codes(worst)
    assert worst["o"] <= 1.0


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 128)])
def test_kda_gate_per_head_widths(torch_cuda, orc, dk, dv):
    """Per-channel (KDA) gate on per-head widths: the gate vector scales each
    key row of the tile before the delta update.  Three teacher-forced steps,
    then the identity rule with a gate vector of ones."""
    from types import SimpleNamespace
    say("case KDA gate, per-head widths", dk, dv)
    rng = np.random.default_rng(300 + dk)
    H, B = 8, 6
    cfg = SimpleNamespace(gate=1, unit=0, window=0)
    wl = SimpleNamespace(B=B, H=H, dk=dk, dv=dv, cfg=cfg, bits=np.array([4, 6, 8, 16, 6, 4, 8, 6], np.int32),
                         row_weight=np.clip(np.exp(rng.normal(0, 1.15, (H, dk))), 0.1, 10).astype(np.float32))
    P = Pair(orc, wl, n_slots=B + 1)
    slots = rng.permutation(B + 1)[:B]
    prof = np.exp(rng.normal(0, 1.5, (1, H, dk, 1))) * np.exp(rng.normal(0, 1.5, (1, H, 1, dv)))
    P.store(slots, (0.1 * rng.standard_normal((B, H, dk, dv)) * prof).astype(np.float32))
    f = lambda x: x.astype(np.float32)
    worst = new_agg()
    for t in range(3):
        img = P.image()
        ref = orc.OraclePool(B + 1, H, dk, dv, wl.bits, wl.row_weight, 1, 0, 0, image=img)
        q = rng.standard_normal((B, H, dk)); q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k = rng.standard_normal((B, H, dk)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
        v = rng.standard_normal((B, H, dv))
        a = 2.0 ** (-1.0 / (10.0 ** rng.uniform(0, 4, (B, H, dk))))
        b = rng.uniform(0.05, 0.95, (B, H))
        o = P.gpu_step(slots, f(q), f(k), f(v), f(a), f(b))
        o_ref = ref.step(slots, f(q), f(k), f(v), f(a), f(b))
        r = compare_codes(orc, ref, P.image(), ref.img, slots)
        add_agg(worst, r, readout_ok(o, o_ref))
    say("  KDA %dx%d: code mismatch %d of %d (max |dQ| %d), pivot mismatch %d of %d, readout %.3f"
        % (dk, dv, worst["mism"], worst["codes"], worst["maxd"], worst["piv_mism"], worst["piv"], worst["o"]))
    _assert_codes(worst)
    assert worst["o"] <= 1.0
    before = P.image()
    q = f(rng.standard_normal((B, H, dk)))
    k = f(rng.standard_normal((B, H, dk)))
    v = f(rng.standard_normal((B, H, dv)))
    P.gpu_step(slots, q, k, v, np.ones((B, H, dk), np.float32), np.zeros((B, H), np.float32))
    np.testing.assert_array_equal(P.image(), before)


@pytest.mark.parametrize("dk,dv,gate,unit", [(128, 128, 0, 0), (128, 128, 1, 0), (128, 128, 1, 1), (128, 64, 1, 1)])
def test_zero_gate(torch_cuda, orc, dk, dv, gate, unit):
    """A gate of zero (a full forget) on quantized and binary16 pivot units:
    S' = k delta^T there.  GDN: whole heads at a = 0, one of them with b = 0 too
    (the state becomes zero: codes 0, scales 1); KDA: zero channels in every
    width.  Two teacher-forced steps against the oracle."""
    from types import SimpleNamespace
    say("case zero gate", dk, dv, "KDA" if gate else "GDN", "rows" if unit else "heads")
    rng = np.random.default_rng(500 + 10 * gate + unit + dv)
    H, B = 8, 5
    cfg = SimpleNamespace(gate=gate, unit=unit, window=0)
    if unit:
        bits = _row_width_patterns(dk, rng)
    else:
        bits = np.array([4, 6, 8, 16, 6, 4, 8, 6], np.int32)
    wl = SimpleNamespace(B=B, H=H, dk=dk, dv=dv, cfg=cfg, bits=bits,
                         row_weight=np.clip(np.exp(rng.normal(0, 1.15, (H, dk))), 0.1, 10).astype(np.float32))
    P = Pair(orc, wl, n_slots=B)
    slots = np.arange(B)
    prof = np.exp(rng.normal(0, 1.5, (1, H, dk, 1))) * np.exp(rng.normal(0, 1.5, (1, H, 1, dv)))
    P.store(slots, (0.1 * rng.standard_normal((B, H, dk, dv)) * prof).astype(np.float32))
    f = lambda x: x.astype(np.float32)
    worst = new_agg()
    for t in range(2):
        img = P.image()
        ref = orc.OraclePool(B, H, dk, dv, np.asarray(bits).reshape(-1), wl.row_weight, gate, unit, 0, image=img)
        q = rng.standard_normal((B, H, dk)); q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k = rng.standard_normal((B, H, dk)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
        v = rng.standard_normal((B, H, dv))
        b = rng.uniform(0.05, 0.95, (B, H))
        if gate:
            a = 2.0 ** (-1.0 / (10.0 ** rng.uniform(0, 4, (B, H, dk))))
            a[rng.uniform(size=a.shape) < 0.1] = 0.0
        else:
            a = rng.uniform(0.9, 1.0, (B, H))
            a[:, [1, 3, 6]] = 0.0                       # a 6-bit, the pivot and an 8-bit head
            b[0, 1] = 0.0                               # a = b = 0: the state becomes zero
        o = P.gpu_step(slots, f(q), f(k), f(v), f(a), f(b))
        o_ref = ref.step(slots, f(q), f(k), f(v), f(a), f(b))
        post = P.image()
        assert np.isfinite(o).all()
        r = compare_codes(orc, ref, post, ref.img, slots)
        add_agg(worst, r, readout_ok(o, o_ref))
        if not gate:                                    # the reset head: every code 0, every scale 1
            Qg, sg, cg, _ = ref.decode_tile(0, 1, post)
            assert not np.any(Qg) and np.all(sg == 0x3F80) and np.all(cg == 0x3F80)   # bf16 1.0
    say("  zero gate: code mismatch %d of %d (max |dQ| %d), scale mismatch %d of %d, pivot mismatch %d of %d, "
        "readout %.3f" % (worst["mism"], worst["codes"], worst["maxd"], worst["scale_mism"], worst["scales"],
                          worst["piv_mism"], worst["piv"], worst["o"]))
    _assert_codes(worst)
    assert worst["o"] <= 1.0


@pytest.mark.parametrize("unit", [0, 1])
def test_max_heads(torch_cuda, orc, unit):
    """The largest head count the descriptor accepts (4,096 heads, d = 64):
    header tables, tile offsets and the grid at their limit.  One step with the
    KDA gate, checked against the oracle on a sample of heads."""
    from types import SimpleNamespace
    say("case max heads", "rows" if unit else "heads")
    rng = np.random.default_rng(700 + unit)
    H, B, dk, dv = 4096, 2, 64, 64
    cfg = SimpleNamespace(gate=1, unit=unit, window=0)
    bits = rng.choice([4, 6, 8, 16], (H, dk) if unit else H, p=[0.3, 0.5, 0.18, 0.02]).astype(np.int32)
    wl = SimpleNamespace(B=B, H=H, dk=dk, dv=dv, cfg=cfg, bits=bits,
                         row_weight=np.clip(np.exp(rng.normal(0, 1.15, (H, dk))), 0.1, 10).astype(np.float32))
    P = Pair(orc, wl, n_slots=B)
    slots = np.arange(B)
    P.store(slots, (0.1 * rng.standard_normal((B, H, dk, dv))).astype(np.float32))
    np.testing.assert_array_equal(P.image(), P.ref.img)
    f = lambda x: x.astype(np.float32)
    q = rng.standard_normal((B, H, dk)); q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.standard_normal((B, H, dk)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, H, dv))
    a = rng.uniform(0.5, 1.0, (B, H, dk))
    b = rng.uniform(0.05, 0.95, (B, H))
    img = P.image()
    o = P.gpu_step(slots, f(q), f(k), f(v), f(a), f(b))
    ref = orc.OraclePool(B, H, dk, dv, np.asarray(bits).reshape(-1), wl.row_weight, 1, unit, 0, image=img)
    o_ref = ref.step(slots, f(q), f(k), f(v), f(a), f(b))
    heads = sorted(set(rng.choice(H, 64, replace=False).tolist()) | {0, H - 1})
    r = compare_codes(orc, ref, P.image(), ref.img, slots, heads=heads)
    say("  max heads: code mismatch %d of %d (max |dQ| %d), pivot mismatch %d of %d, readout %.3f"
        % (r["mism"], r["codes"], r["maxd"], r["piv_mism"], r["piv"], readout_ok(o, o_ref)))
    _assert_codes(r)
    assert readout_ok(o, o_ref) <= 1.0


def test_step_from_fresh_pool(torch_cuda, orc):
    """A step straight after pool creation (every state zero: codes 0, scales
    1), GDN head mix, two teacher-forced steps."""
    say("case fresh pool")
    wl = Workload("C2", B=8)
    P = Pair(orc, wl)
    slots = np.arange(8)
    np.testing.assert_array_equal(P.image(), P.ref.img)
    r = _teacher_forced(orc, wl, P, slots, 2)
    say("  fresh pool: code mismatch %d of %d (max |dQ| %d), pivot mismatch %d of %d, readout %.3f"
        % (r["mism"], r["codes"], r["maxd"], r["piv_mism"], r["piv"], r["o"]))
    _assert_codes(r)
    assert r["o"] <= 1.0


def test_empty_and_out_of_range(torch_cuda, orc):
    say("case edges")
    torch = torch_cuda
    wl = Workload("C1", B=4)
    P = Pair(orc, wl)
    P.store(np.arange(4), wl.state(np.arange(4)))
    before = P.image()
    z = torch.empty(0, dtype=torch.int32, device="cuda")
    e = torch.empty(0, dtype=torch.float32, device="cuda")
    P.stq.stq_decode_step(P.pool, z, e, e, e, e, e, e)
    P.stq.stq_pool_store(P.pool, z, e)
    np.testing.assert_array_equal(P.image(), before)
    # a slot index outside the pool is skipped on the device
    q, k, v, a, b = wl.token(0, 2)
    P.gpu_step(np.array([7, 99]), q, k, v, a, b)
    np.testing.assert_array_equal(P.image(), before)


def _cache_view(ref, img, slot, h):
    """(count, G[W], K[W][dk], U[W][dv]) of one tile's window cache."""
    offs, sb = ref.head_offsets()
    stride = 256 + 4 * ref.W * (ref.dk + ref.dv)
    base = ref.hdr_bytes() + ref.n_slots * sb + (slot * ref.H + h) * stride
    c = img[base: base + stride]
    cnt = int(c[:4].view(np.int32)[0])
    G = c[4: 4 + 4 * ref.W].view(np.float32)
    K = c[256: 256 + 4 * ref.W * ref.dk].view(np.float32).reshape(ref.W, ref.dk)
    U = c[256 + 4 * ref.W * ref.dk: stride].view(np.float32).reshape(ref.W, ref.dv)
    return cnt, G, K, U


@pytest.mark.parametrize("W,T,mix", [(16, 19, False), (4, 9, False), (8, 10, True), (32, 33, False)])
def test_window_teacher_forced(torch_cuda, orc, W, T, mix):
    """Window mode (base frozen inside the window, fp32 cache, fold after token
    W): the oracle steps from the GPU's bytes at every token.  The C5 pool is
    all 4-bit; `mix` gives it the GDN head mix (4/6/8-bit and a binary16 pivot
    head) so that every width's window path runs; W = 32 is the largest window."""
    say("case window", W, T, "mix" if mix else "4-bit")
    wl = Workload("C5", B=24)
    if mix:
        wl.bits = Workload("C2", H=wl.H).bits
    P = Pair(orc, wl, n_slots=26, window=W)
    slots = np.random.default_rng(3).permutation(26)[:24]
    P.store(slots, wl.state(slots))
    agg = new_agg()
    worst_o = worst_u = 0.0
    for t in range(T):
        img = P.image()
        ref = orc.OraclePool(26, wl.H, wl.dk, wl.dv, wl.bits, wl.row_weight, window=W, image=img)
        q, k, v, a, b = wl.token(t, 24)
        o = P.gpu_step(slots, q, k, v, a, b)
        o_ref = ref.step(slots, q, k, v, a, b)
        post = P.image()
        worst_o = max(worst_o, readout_ok(o, o_ref))
        for s in slots[:6]:
            for h in range(wl.H):
                cg, Gg, Kg, Ug = _cache_view(ref, post, int(s), h)
                cr, Gr, Kr, Ur = _cache_view(ref, ref.img, int(s), h)
                assert cg == cr == (t + 1) % W
                np.testing.assert_array_equal(Gg[:cg], Gr[:cr])
                np.testing.assert_array_equal(Kg[:cg], Kr[:cr])
                if cg:
                    scale = np.abs(Ur[:cg]).max()
                    worst_u = max(worst_u, float(np.abs(Ug[:cg] - Ur[:cr]).max() / scale))
        if (t + 1) % W == 0:                  # a fold happened: compare the new base
            r = compare_codes(orc, ref, post, ref.img, slots)
            add_agg(agg, r)
        else:                                 # base frozen: bytes of the tiles unchanged
            for s in slots[:4]:
                for h in range(wl.H):
                    np.testing.assert_array_equal(ref.tile_view(int(s), h, post), ref.tile_view(int(s), h, img))
    say("  window W=%d: readout %.3f, cache u rel err %.2e, fold code mismatch %d of %d (max |dQ| %d)"
        % (W, worst_o, worst_u, agg["mism"], agg["codes"], agg["maxd"]))
    assert worst_o <= 1.0
    assert worst_u <= 1e-4
    _assert_codes(agg)


def test_window_flush(torch_cuda, orc):
    say("case window flush")
    W = 16
    wl = Workload("C5", B=8)
    P = Pair(orc, wl, window=W)
    slots = np.arange(8)
    P.store(slots, wl.state(slots))
    before = P.image()
    P.stq.stq_window_flush(P.pool, P.slots_t(slots))         # empty windows: no-op
    np.testing.assert_array_equal(P.image(), before)
    for t in range(5):
        P.gpu_step(slots, *wl.token(t, 8))
    img = P.image()
    ref = orc.OraclePool(8, wl.H, wl.dk, wl.dv, wl.bits, wl.row_weight, window=W, image=img)
    part = np.array([1, 4, 6])
    P.stq.stq_window_flush(P.pool, P.slots_t(part))
    ref.window_flush(part)
    post = P.image()
    r = compare_codes(orc, ref, post, ref.img, part)
    _assert_codes(r)
    for s in part:
        assert _cache_view(ref, post, int(s), 0)[0] == 0
    for s in (0, 2, 3, 5, 7):                                   # untouched slots keep their window
        assert _cache_view(ref, post, int(s), 0)[0] == 5
        np.testing.assert_array_equal(ref.tile_view(int(s), 0, post), ref.tile_view(int(s), 0, img))


# ---- compensator tokens (window mode) ----

def _planted_state(wl, slots, seed):
    """Pool states with three outlier key rows per tile (x60, x40, x25)."""
    rng = np.random.default_rng(seed)
    S = wl.state(slots).copy()
    for c in range(S.shape[0]):
        for h in range(S.shape[1]):
            for r, f in zip(rng.choice(wl.dk, 3, replace=False), (60.0, 40.0, 25.0)):
                S[c, h, r] *= f
    return S


def _comp_pool(orc, W, C, B=12, n_slots=14):
    wl = Workload("C5", B=B)
    wl.bits = Workload("C2", H=wl.H).bits        # 4/6/8-bit heads and a binary16 pivot head
    return wl, Pair(orc, wl, n_slots=n_slots, window=W, n_comp=C)


def test_comp_store_fetch_bit_exact(torch_cuda, orc):
    """Ingest with compensators: the C largest rows kept exactly, R of the
    residual; pool image (tiles, scales, caches with the compensator rows and
    values) bit-exact with the oracle's, and fetch adds the rows back."""
    say("case compensators store/fetch")
    import torch
    wl, P = _comp_pool(orc, 8, 4)
    slots = np.random.default_rng(11).permutation(P.n_slots)[:wl.B]
    S = _planted_state(wl, slots, 5)
    P.store(slots, S)
    np.testing.assert_array_equal(P.image(), P.ref.img)
    F = torch.empty((len(slots), wl.H, wl.dk, wl.dv), dtype=torch.float32, device="cuda")
    P.stq.stq_pool_fetch(P.pool, P.slots_t(slots), F)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(F.cpu().numpy(), P.ref.fetch(slots))


@pytest.mark.parametrize("W,C,T", [(8, 3, 17), (4, 8, 9), (16, 4, 17), (24, 8, 25)])
def test_comp_window_teacher_forced(torch_cuda, orc, W, C, T):
    """Window steps with compensator tokens riding the cache path: readout and
    cached u every token, and at each fold the new compensator rows (same
    rows; values to binary32 rounding) and the new base's codes to the bar."""
    say("case compensators window", W, C, T)
    wl, P = _comp_pool(orc, W, C)
    slots = np.random.default_rng(12).permutation(P.n_slots)[:wl.B]
    P.store(slots, _planted_state(wl, slots, 6))
    agg = new_agg()
    worst_o = worst_u = worst_c = 0.0
    for t in range(T):
        img = P.image()
        ref = orc.OraclePool(P.n_slots, wl.H, wl.dk, wl.dv, wl.bits, wl.row_weight, window=W, image=img,
                             n_comp=C)
        q, k, v, a, b = wl.token(t, len(slots))
        o = P.gpu_step(slots, q, k, v, a, b)
        o_ref = ref.step(slots, q, k, v, a, b)
        post = P.image()
        worst_o = max(worst_o, readout_ok(o, o_ref))
        for s in slots[:5]:
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
        if (t + 1) % W == 0:
            r = compare_codes(orc, ref, post, ref.img, slots)
            add_agg(agg, r)
    say("  W=%d C=%d: readout %.3f, cache u %.2e, compensators %.2e, fold code mismatch %d of %d (max |dQ| %d)"
        % (W, C, worst_o, worst_u, worst_c, agg["mism"], agg["codes"], agg["maxd"]))
    assert worst_o <= 1.0
    assert worst_u <= 1e-4
    assert worst_c <= 1e-5
    _assert_codes(agg)


@pytest.mark.parametrize("dk,dv,W,C", [(64, 64, 8, 0), (64, 128, 16, 2), (128, 64, 8, 2)])
def test_window_shapes(torch_cuda, orc, dk, dv, W, C):
    """Window mode at the other tile shapes, with the head mix (4/6/8-bit and a
    binary16 pivot head) and, where C > 0, compensator rows (d_k = 64, W = 16,
    C = 2 takes the fold's 32-entry bound): teacher-forced through one fold and
    a token past it, held to the bars of the d = 128 window tests."""
    say("case window shape", dk, dv, W, C)
    B, H = 6, 8
    wl = Workload("C2", B=B, H=H)
    wl.dk, wl.dv = dk, dv
    wl.row_weight = wl.row_weight[:, :dk].copy()
    wl.bits = np.array([4, 6, 8, 16, 6, 4, 8, 6], np.int32)
    rng = np.random.default_rng(dk * 3 + dv + W + C)
    P = Pair(orc, wl, n_slots=B + 2, window=W, n_comp=C)
    slots = rng.permutation(B + 2)[:B]
    S = (rng.standard_normal((B, H, dk, dv)) * np.exp(rng.normal(0, 1.5, (1, H, dk, 1)))).astype(np.float32)
    for c in range(B):
        for h in range(H):
            for r, f in zip(rng.choice(dk, 2, replace=False), (50.0, 30.0)):
                S[c, h, r] *= f
    P.store(slots, S)
    np.testing.assert_array_equal(P.image(), P.ref.img)
    f = lambda x: x.astype(np.float32)
    agg = new_agg()
    worst_o = worst_u = 0.0
    for t in range(W + 1):
        img = P.image()
        ref = orc.OraclePool(B + 2, H, dk, dv, wl.bits, wl.row_weight, window=W, image=img, n_comp=C)
        q = rng.standard_normal((B, H, dk)); q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k = rng.standard_normal((B, H, dk)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
        v = rng.standard_normal((B, H, dv))
        a = rng.uniform(0.9, 1, (B, H)); b = rng.uniform(0, 1, (B, H))
        o = P.gpu_step(slots, f(q), f(k), f(v), f(a), f(b))
        o_ref = ref.step(slots, f(q), f(k), f(v), f(a), f(b))
        post = P.image()
        worst_o = max(worst_o, readout_ok(o, o_ref))
        for s in slots:
            for h in range(H):
                cg, Gg, Kg, Ug, ig, vg = ref.cache_view(int(s), h, post)
                cr, Gr, Kr, Ur, ir, vr = ref.cache_view(int(s), h)
                assert cg == cr == (t + 1) % W
                np.testing.assert_array_equal(Gg[:cg], Gr[:cr])
                np.testing.assert_array_equal(Kg[:cg], Kr[:cr])
                if cg:
                    worst_u = max(worst_u, float(np.abs(Ug[:cg] - Ur[:cr]).max() / np.abs(Ur[:cr]).max()))
                np.testing.assert_array_equal(ig, ir)
        if (t + 1) % W == 0:
            add_agg(agg, compare_codes(orc, ref, post, ref.img, slots))
    say("  window %dx%d W=%d C=%d: readout %.3f, cache u %.2e, fold %s"
        % (dk, dv, W, C, worst_o, worst_u, agg_text(agg)))
    assert worst_o <= 1.0
    assert worst_u <= 1e-4
    _assert_codes(agg)


def test_comp_flush(torch_cuda, orc):
    say("case compensators flush")
    W, C = 16, 2
    wl, P = _comp_pool(orc, W, C, B=8, n_slots=8)
    slots = np.arange(8)
    P.store(slots, _planted_state(wl, slots, 7))
    for t in range(5):
        P.gpu_step(slots, *wl.token(t, 8))
    img = P.image()
    ref = orc.OraclePool(8, wl.H, wl.dk, wl.dv, wl.bits, wl.row_weight, window=W, image=img, n_comp=C)
    part = np.array([0, 3, 5])
    P.stq.stq_window_flush(P.pool, P.slots_t(part))
    ref.window_flush(part)
    post = P.image()
    _assert_codes(compare_codes(orc, ref, post, ref.img, part))
    for s in part:
        for h in range(wl.H):
            cg, _, _, _, ig, vg = ref.cache_view(int(s), h, post)
            cr, _, _, _, ir, vr = ref.cache_view(int(s), h)
            assert cg == cr == 0
            np.testing.assert_array_equal(ig, ir)
            if (ir >= 0).any():
                assert np.abs(vg - vr).max() <= 1e-5 * np.abs(vr).max()
