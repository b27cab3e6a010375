"""GPU parity of the prefill ingest (stq_prefill) against the oracle, through the C ABI.

The oracle runs the per-token recurrence in binary64 and writes R(fl32(S_T));
the kernel runs the chunkwise form in binary32 and writes R of its own binary32
S_T.  Bar (written here):
  - readout: |o - o_ref| <= 1e-3 (|o_ref| + 0.01 max|o_ref|) per (token, head);
  - final state, every element: |D(tile) - S_T| <= half the tile's own code step
    sigma_i c_j (binary16 pivots: half an ulp) + 1e-4 max|S_T| of the tile, i.e.
    each code is the nearest one to the exact state up to the binary32 error of
    the evaluation;
  - codes against the oracle's R(fl32(S_T)): every difference <= 1 step and at
    most 1e-4 of the codes differ (only codes whose exact value lies within
    that binary32 error of a rounding boundary, or rows whose bf16 scale does,
    can; the error is about (T/L)(d_k + L) unit roundoffs of the tile's scale,
    1e-5 at T = 300, so a code sits that close to a boundary about once in 1e5:
    0-27 differing codes of up to 2.5 million were measured);
  - row and column scales (as the steps they define) each within one bf16
    step, at most 1e-3 of them differing: a scale's input is a row or column
    absmax, which carries the evaluation's error relative to the tile's scale
    while being smaller than it, and sits on a 2^-8-relative bf16 grid, so it
    lands within that error of a rounding boundary more often than a code
    does (measured: at most 2 of 15,872);
  - empty requests and requests of identity tokens leave their tiles' bytes
    (window pools: their folded windows are compared like the rest).
"""
import numpy as np
import pytest

from gpu_util import Pair, agg_text, compare_codes, readout_ok, say
from workloads import Workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available()
    return torch


def _run(P, wl, slots, lens, edit=None, prompts=None):
    import torch
    dev = lambda x: torch.as_tensor(x, device="cuda")
    ss, q, k, v, a, b = wl.prompts(lens) if prompts is None else prompts
    if edit:
        edit(ss, q, k, v, a, b)
    pre = P.image()
    ref = P.orc.OraclePool(P.n_slots, wl.H, wl.dk, wl.dv, np.asarray(wl.bits).reshape(-1), wl.row_weight,
                           P.ref.gate, P.ref.unit, P.ref.W, image=pre, n_comp=P.ref.C)
    T = int(ss[-1])
    o = torch.full((T, wl.H, wl.dv), float("nan"), dtype=torch.float32, device="cuda")
    P.stq.stq_prefill(P.pool, P.slots_t(slots), dev(ss), dev(q), dev(k), dev(v), dev(a), dev(b), o)
    torch.cuda.synchronize()
    o_ref, S_fin = ref.prefill(slots, ss, q, k, v, a, b, final_state=True)
    return pre, P.image(), ref, o.cpu().numpy(), o_ref, S_fin, ss


def _state_ok(orc, ref, img, slots, S_fin, moved):
    """Worst ratio of |D(tile) - S_T| to its bound over the tiles that moved."""
    D = orc.OraclePool(ref.n_slots, ref.H, ref.dk, ref.dv, ref.bits, ref.wt, ref.gate, ref.unit, ref.W, image=img,
                       n_comp=ref.C).fetch(slots)
    worst = 0.0
    for c, s in enumerate(slots):
        if not moved[c]:
            continue
        for h in range(ref.H):
            S = S_fin[c, h]
            Q, sg, cs, nb = ref.decode_tile(int(s), h, img)
            eps = 1e-4 * np.abs(S).max()
            # per row: half a code step sigma_i c_j, binary16 pivot rows half an ulp
            sig = (sg.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
            col = (cs.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
            half = 0.5 * sig[:, None] * col[None, :] * (1 + 1e-6)
            piv = np.asarray(nb) == 16
            half[piv] = (np.abs(S) * 2.0 ** -11 + 2.0 ** -25)[piv]
            err = np.abs(D[c, h].astype(np.float64) - S)
            worst = max(worst, float((err / (half + eps)).max()))
    return worst


CODE_MAX = 1e-4
SCALE_MAX = 1e-3


def _assert_prefill_codes(res):
    assert res["maxd"] <= 1
    assert res["mism"] <= CODE_MAX * max(res["codes"], 1)
    assert res["piv_bad"] == 0
    assert res["scale_mism"] <= SCALE_MAX * max(res["scales"], 1)
    assert res["scale_steps"] <= 1


def _check(P, wl, slots, lens, pre, img, ref, o, o_ref, S_fin, ss, moved):
    T = int(ss[-1])
    if T:
        r = readout_ok(o.reshape(T, 1, wl.H, wl.dv), o_ref.reshape(T, 1, wl.H, wl.dv))
        say("  readout worst ratio %.3g" % r)
        assert r <= 1.0
    w = _state_ok(P.orc, ref, img, slots, S_fin, moved)
    say("  state worst ratio %.3g" % w)
    assert w <= 1.0
    # a window pool folds every listed slot's open window first: those tiles all change
    mv = [s for c, s in enumerate(slots) if moved[c] or ref.W]
    if mv:
        res = compare_codes(P.orc, ref, img, ref.img, mv)
        say("  " + agg_text(res))
        _assert_prefill_codes(res)
    H = wl.H
    for c, s in enumerate(slots):
        if not moved[c] and not ref.W:
            for h in range(H):
                assert np.array_equal(ref.tile_view(int(s), h, img), ref.tile_view(int(s), h, pre)), (c, h)


@pytest.mark.parametrize("key,H,lens", [
    ("C2", 32, [33, 0, 1, 100, 32, 7]),          # GDN head mix with a binary16 head, ragged tails
    ("C1", 2, [70, 3, 0, 64, 31]),               # 64 x 64 tiles, 8-bit
    ("C3", 8, [257, 5]),                         # persistent outlier rows and columns, long prompt
])
def test_prefill_parity(torch_cuda, orc, key, H, lens):
    say("case prefill", key, H, lens)
    B = len(lens)
    wl = Workload(key, B=B, H=H)
    P = Pair(orc, wl, n_slots=B + 3)
    slots = np.random.default_rng(B).permutation(B + 3)[:B].astype(np.int32)   # distinct slots
    P.store(slots, wl.state(slots))
    out = _run(P, wl, slots, lens)
    _check(P, wl, slots, lens, *out, moved=[L > 0 for L in lens])


@pytest.mark.parametrize("dk,dv", [(64, 128), (128, 64)])
def test_prefill_other_shapes(torch_cuda, orc, dk, dv):
    say("case prefill shape", dk, dv)
    wl = Workload("C2", B=3, H=8)
    wl.dk, wl.dv = dk, dv
    wl.row_weight = wl.row_weight[:, :dk].copy()
    wl.bits = np.array([4, 6, 8, 16, 6, 4, 8, 6], np.int32)
    P = Pair(orc, wl)
    slots = np.arange(3, dtype=np.int32)
    rng = np.random.default_rng(dk * 3 + dv)
    S = (rng.standard_normal((3, 8, dk, dv)) * np.exp(rng.normal(0, 1.5, (1, 8, dk, 1)))).astype(np.float32)
    P.store(slots, S)
    lens = [45, 16, 1]
    out = _run(P, wl, slots, lens)
    _check(P, wl, slots, lens, *out, moved=[True] * 3)


def test_prefill_fresh_pool_and_identity(torch_cuda, orc):
    """From the all-zero state of a fresh pool; one request of identity tokens only."""
    say("case prefill fresh + identity")
    wl = Workload("C2", B=3, H=32)
    P = Pair(orc, wl)
    slots = np.array([2, 0, 1], np.int32)
    lens = [40, 12, 9]

    def edit(ss, q, k, v, a, b):
        a[ss[1]:ss[2]] = 1.0
        b[ss[1]:ss[2]] = 0.0

    out = _run(P, wl, slots, lens, edit)
    _check(P, wl, slots, lens, *out, moved=[True, False, True])


def test_prefill_zero_gates(torch_cuda, orc):
    """Zero gates inside a chunk forget everything before them (no division by
    a gate product anywhere); b = 0 tokens in between."""
    say("case prefill zero gates")
    wl = Workload("C2", B=2, H=8)
    P = Pair(orc, wl)
    slots = np.array([0, 1], np.int32)
    P.store(slots, wl.state(slots))
    lens = [50, 20]

    def edit(ss, q, k, v, a, b):
        a[3, :] = 0.0
        a[40, :4] = 0.0
        b[41:45, :] = 0.0
        a[ss[1] + 19, :] = 0.0        # the last token of a request

    out = _run(P, wl, slots, lens, edit)
    _check(P, wl, slots, lens, *out, moved=[True, True])


@pytest.mark.parametrize("W,C", [(16, 0), (8, 4)])
def test_prefill_window_pool(torch_cuda, orc, W, C):
    """Window pools: slots with open windows (folded first) and compensator rows
    (part of the start state, taken again from the final state)."""
    say("case prefill window pool", W, C)
    wl = Workload("C5", B=4, H=8)
    P = Pair(orc, wl, n_slots=5, window=W, n_comp=C)
    slots = np.array([3, 0, 4, 1], np.int32)
    P.store(slots, wl.state(slots))
    for t in range(3):                                  # leave a window open in every slot
        q, k, v, a, b = wl.token(t, n=4)
        P.gpu_step(slots, q, k, v, a, b)
    lens = [37, 0, 5, 64]
    out = _run(P, wl, slots, lens)
    pre, img, ref = out[0], out[1], out[2]
    _check(P, wl, slots, lens, *out, moved=[L > 0 for L in lens])
    # compensator rows: the same rows, values within the evaluation error; windows empty
    for c, s in enumerate(slots):
        for h in range(wl.H):
            g, r = ref.cache_view(int(s), h, img), ref.cache_view(int(s), h, ref.img)
            assert g[0] == 0 and r[0] == 0
            if C:
                assert np.array_equal(g[4], r[4]), (c, h)
                assert np.abs(g[5] - r[5]).max() <= 1e-4 * np.abs(r[5]).max(), (c, h)


@pytest.mark.parametrize("dk,dv,zero", [(128, 128, False), (64, 128, True), (64, 64, True), (128, 64, False)])
def test_prefill_per_channel_gate(torch_cuda, orc, dk, dv, zero):
    """Per-channel (KDA) gates on per-head widths, with the KDA half-life law:
    the chunkwise form; with zero gates (when asked) a request's tokens from
    the chunk that holds one run token by token: head 0 of the first request
    from its first chunk, the other heads from its second (the first chunk
    chunkwise), head 2 of the last request from its first; tiny nonzero gates
    whose chunk product falls below 2^-60 do the same (head 3 of the first
    request would, from its third chunk)."""
    import dataclasses
    say("case prefill per-channel gate", dk, dv, zero)
    wl = Workload("C4", B=3, H=8)
    wl.cfg = dataclasses.replace(wl.cfg, unit=0)
    wl.dk, wl.dv = dk, dv
    wl.row_weight = wl.row_weight[:, :dk].copy()
    wl.r_prof, wl.c_prof = wl.r_prof[:, :dk].copy(), wl.c_prof[:, :dv].copy()
    wl.half_life = wl.half_life[:, :dk].copy()
    wl.bits = np.array([4, 6, 8, 16, 6, 4, 8, 6], np.int32)
    P = Pair(orc, wl, n_slots=4)
    slots = np.array([2, 0, 3], np.int32)
    P.store(slots, wl.state(slots))
    lens = [70, 0, 33]

    def edit(ss, q, k, v, a, b):
        if zero:
            a[5, 0, :7] = 0.0
            a[40, :, :7] = 0.0
            a[ss[2] + 31, 2, :] = 0.0
            a[64:70, 3, 10:20] = 1e-4     # nonzero, but the chunk's product (1e-24) is below the form's floor

    out = _run(P, wl, slots, lens, edit if zero else None)
    _check(P, wl, slots, lens, *out, moved=[L > 0 for L in lens])


def test_prefill_unsupported_and_empty(torch_cuda, orc):
    import torch
    import quantized_linear_attention_amd as stq
    say("case prefill unsupported pools, n = 0")
    f = lambda *s: torch.zeros(s, dtype=torch.float32, device="cuda")
    for key in ("C4",):                            # per-key-row units: one request, no tokens
        wl = Workload(key, B=1, H=2)
        P = Pair(orc, wl, n_slots=1)
        P.store(np.array([0]), wl.state(np.array([0])))
        pre = P.image()
        ss = torch.zeros(2, dtype=torch.int32, device="cuda")      # an empty request (buffers for one token)
        H, dk, dv = wl.H, wl.dk, wl.dv
        stq.stq_prefill(P.pool, P.slots_t([0]), ss, f(H * dk), f(H * dk), f(H * dv), f(H * dk), f(H), f(H * dv))
        assert np.array_equal(P.image(), pre)
    wl = Workload("C2", B=1, H=2)
    P = Pair(orc, wl, n_slots=1)
    pre = P.image()
    ss = torch.zeros(1, dtype=torch.int32, device="cuda")
    stq.stq_prefill(P.pool, P.slots_t(np.zeros(0, np.int32)), ss, f(0), f(0), f(0), f(0), f(0), f(0))
    assert np.array_equal(P.image(), pre)


@pytest.mark.parametrize("key,gate", [("C2", 0), ("C4", 1)])
def test_prefill_states_against_recurrence(torch_cuda, orc, key, gate):
    """stq_prefill_states on plain binary32 states: final states within the
    binary32 evaluation error (1e-4 of the tile's largest |S_T|) of the
    oracle's binary64 recurrence, readouts to the bar above."""
    import torch
    say("case prefill states", key, gate)
    wl = Workload(key, B=3, H=8)
    lens = [50, 0, 17]
    slots = np.arange(3, dtype=np.int32)
    S0 = wl.state(slots)
    ss, q, k, v, a, b = wl.prompts(lens)
    dev = lambda x: torch.as_tensor(x, device="cuda")
    S = dev(S0).contiguous()
    o = torch.zeros((int(ss[-1]), wl.H, wl.dv), dtype=torch.float32, device="cuda")
    import quantized_linear_attention_amd as stq
    stq.stq_prefill_states(S, dev(ss), dev(q), dev(k), dev(v), dev(a), dev(b), o, gate_kind=gate)
    torch.cuda.synchronize()
    # the oracle's recurrence from the same binary32 states: a pool of binary16
    # heads only would round them, so run its update directly
    T_all = []
    for c in range(3):
        Sx = S0[c].astype(np.float64)
        for t in range(ss[c], ss[c + 1]):
            for h in range(wl.H):
                ah = a[t, h] if gate else a[t, h:h + 1]
                Sx[h], oo = orc.update_f64(Sx[h], q[t, h], k[t, h], v[t, h], ah, b[t, h])
                T_all.append((t, h, oo))
        Sg = S.cpu().numpy()[c].astype(np.float64)
        for h in range(wl.H):
            assert np.abs(Sg[h] - Sx[h]).max() <= 1e-4 * np.abs(Sx[h]).max(), (c, h)
    og = o.cpu().numpy()
    o_ref = np.zeros(og.shape)
    for t, h, oo in T_all:
        o_ref[t, h] = oo
    assert readout_ok(og.reshape(-1, 1, wl.H, wl.dv), o_ref.reshape(-1, 1, wl.H, wl.dv)) <= 1.0
    assert np.array_equal(S.cpu().numpy()[1], S0[1])          # no tokens: untouched


def test_prefill_states_per_key_row_pool(torch_cuda, orc):
    """Per-key-row (C4) pools through fetch -> stq_prefill_states -> store,
    against the oracle's prefill of the same pool."""
    import torch
    import quantized_linear_attention_amd as stq
    say("case prefill states C4 pool")
    wl = Workload("C4", B=3, H=8)
    P = Pair(orc, wl, n_slots=4)
    slots = np.array([3, 1, 0], np.int32)
    P.store(slots, wl.state(slots))
    lens = [41, 9, 30]
    ss, q, k, v, a, b = wl.prompts(lens)
    dev = lambda x: torch.as_tensor(x, device="cuda")
    pre = P.image()
    ref = orc.OraclePool(4, wl.H, wl.dk, wl.dv, np.asarray(wl.bits).reshape(-1), wl.row_weight, 1, 1, 0, image=pre)
    S = torch.empty((3, wl.H, wl.dk, wl.dv), dtype=torch.float32, device="cuda")
    sl = P.slots_t(slots)
    o = torch.empty((int(ss[-1]), wl.H, wl.dv), dtype=torch.float32, device="cuda")
    stq.stq_pool_fetch(P.pool, sl, S)
    stq.stq_prefill_states(S, dev(ss), dev(q), dev(k), dev(v), dev(a), dev(b), o, gate_kind=1)
    stq.stq_pool_store(P.pool, sl, S)
    torch.cuda.synchronize()
    o_ref, S_fin = ref.prefill(slots, ss, q, k, v, a, b, final_state=True)
    r = readout_ok(o.cpu().numpy().reshape(-1, 1, wl.H, wl.dv), o_ref.reshape(-1, 1, wl.H, wl.dv))
    say("  readout worst ratio %.3g" % r)
    assert r <= 1.0
    res = compare_codes(orc, ref, P.image(), ref.img, slots)
    say("  " + agg_text(res))
    _assert_prefill_codes(res)


# ---- per-key-row units (unit = key row): stq_prefill straight into the row records ----

def _rows_workload(dk, dv, gate, B, H, seed):
    """Per-key-row widths that reach every run boundary (the C4 proportions, a
    lone quantized row among pivots, one width only, all pivots, random)."""
    from types import SimpleNamespace
    from test_gpu_parity import _row_width_patterns
    rng = np.random.default_rng(seed)
    pats = _row_width_patterns(dk, rng)
    bits = pats[rng.integers(0, len(pats), H)]
    bits[0] = pats[5]                              # the C4 mix
    wl = Workload("C4", B=B, H=H)
    wl.dk, wl.dv = dk, dv
    wl.bits = bits
    wl.row_weight = np.clip(np.exp(rng.normal(0, 1.15, (H, dk))), 0.1, 10).astype(np.float32)
    wl.cfg = SimpleNamespace(**{**wl.cfg.__dict__, "gate": gate, "unit": 1})
    prof = np.exp(rng.normal(0, 1.5, (1, H, dk, 1))) * np.exp(rng.normal(0, 1.5, (1, H, 1, dv)))
    S0 = (0.1 * rng.standard_normal((B, H, dk, dv)) * prof).astype(np.float32)
    return wl, S0


def _rows_prompts(wl, lens, gate, seed):
    rng = np.random.default_rng(seed)
    T, H, dk, dv = sum(lens), wl.H, wl.dk, wl.dv
    ss = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    q = rng.standard_normal((T, H, dk)); q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.standard_normal((T, H, dk)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, dv))
    b = rng.uniform(0.05, 0.95, (T, H))
    a = (2.0 ** (-1.0 / (10.0 ** rng.uniform(0, 4, (T, H, dk))))) if gate else rng.uniform(0.9, 0.9999, (T, H))
    f = lambda x: x.astype(np.float32)
    return ss, f(q), f(k), f(v), f(a), f(b)


@pytest.mark.parametrize("dk,dv,gate", [(128, 128, 1), (128, 128, 0), (64, 128, 1), (128, 64, 1), (64, 64, 0), (64, 64, 1)])
def test_prefill_rows_parity(torch_cuda, orc, dk, dv, gate):
    """Per-key-row pools through stq_prefill (no binary32 staging): ragged
    prompts, tails inside a chunk, an empty request; per-channel (KDA) and
    per-head gates."""
    say("case prefill rows", dk, dv, "KDA" if gate else "GDN")
    B, H = 4, 6
    wl, S0 = _rows_workload(dk, dv, gate, B, H, 900 + dk + dv + gate)
    P = Pair(orc, wl, n_slots=B + 1)
    slots = np.array([4, 0, 2, 1], np.int32)
    P.store(slots, S0)
    lens = [45, 0, 33, 70]
    out = _run(P, wl, slots, lens, prompts=_rows_prompts(wl, lens, gate, 17 + dk + gate))
    _check(P, wl, slots, lens, *out, moved=[L > 0 for L in lens])


def test_prefill_states_gates_one_paths_agree(torch_cuda, orc):
    """With every gate 1 the per-channel chunk form (Gamma = 1: K~ = K^ = K,
    Q~ = Q) performs exactly the scalar-gate chunk form's operations, so the
    two paths must give bit-identical states and readouts."""
    import torch
    import quantized_linear_attention_amd as stq
    say("case prefill states, gates 1: per-channel path against scalar-gate path")
    wl = Workload("C4", B=2, H=8)
    ss, q, k, v, a, b = wl.prompts([100, 37])
    T = int(ss[-1])
    dev = lambda x: torch.as_tensor(np.ascontiguousarray(x), device="cuda")
    S0 = wl.state(np.arange(2)).astype(np.float32)
    S_g, S_k = dev(S0), dev(S0)
    o_g = torch.empty((T, wl.H, wl.dv), dtype=torch.float32, device="cuda")
    o_k = torch.empty_like(o_g)
    stq.stq_prefill_states(S_g, dev(ss), dev(q), dev(k), dev(v), dev(np.ones((T, wl.H), np.float32)), dev(b), o_g,
                           gate_kind=0)
    stq.stq_prefill_states(S_k, dev(ss), dev(q), dev(k), dev(v), dev(np.ones((T, wl.H, wl.dk), np.float32)),
                           dev(b), o_k, gate_kind=1)
    torch.cuda.synchronize()
    assert torch.equal(S_g, S_k)
    assert torch.equal(o_g, o_k)


@pytest.mark.parametrize("unit", [0, 1])
def test_prefill_per_channel_identity(torch_cuda, orc, unit):
    """Per-channel gates: a request whose tokens are all the identity (every
    gate 1, b = 0) leaves its tiles' bytes as they are, next to requests that
    move, on per-head and per-key-row widths."""
    import dataclasses
    say("case prefill per-channel identity, unit", unit)
    wl = Workload("C4", B=3, H=8)
    if unit == 0:
        wl.cfg = dataclasses.replace(wl.cfg, unit=0)
        wl.bits = np.array([4, 6, 8, 16, 6, 4, 8, 6], np.int32)
    P = Pair(orc, wl, n_slots=4)
    slots = np.array([3, 1, 0], np.int32)
    P.store(slots, wl.state(slots))
    lens = [40, 37, 9]

    def edit(ss, q, k, v, a, b):
        a[ss[1]:ss[2]] = 1.0
        b[ss[1]:ss[2]] = 0.0

    out = _run(P, wl, slots, lens, edit)
    _check(P, wl, slots, lens, *out, moved=[True, False, True])


@pytest.mark.parametrize("gate", [1, 0])
def test_prefill_rows_exact_scaling(torch_cuda, orc, gate):
    """Gates of 1/2 and b = 0: the final state is D(tile) times an exact power
    of two in both binary32 and binary64, so the per-key-row refit of the
    kernel must write the oracle's bytes exactly (row and column scales,
    codes in every width, binary16 pivot rows)."""
    say("case prefill rows exact", "KDA" if gate else "GDN")
    B, H, dk, dv = 2, 6, 128, 128
    wl, S0 = _rows_workload(dk, dv, gate, B, H, 950 + gate)
    P = Pair(orc, wl, n_slots=B)
    slots = np.array([1, 0], np.int32)
    P.store(slots, S0)
    lens = [3, 40]
    ss, q, k, v, a, b = _rows_prompts(wl, lens, gate, 5)
    a[:] = 0.5
    b[:] = 0.0
    pre, img, ref, o, o_ref, S_fin, ss2 = _run(P, wl, slots, lens, prompts=(ss, q, k, v, a, b))
    assert not np.array_equal(img, pre)            # the tiles were rewritten
    np.testing.assert_array_equal(img, ref.img)
