"""Helpers shared by the GPU parity tests (marshalling and comparison only)."""
import sys

import numpy as np

from workloads import Workload


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


class Pair:
    """A GPU pool (through the C ABI) and the oracle's pool, same description."""

    def __init__(self, orc, wl, n_slots=None, window=None, n_comp=0):
        import torch
        import quantized_linear_attention_amd as stq
        self.stq, self.orc, self.wl = stq, orc, wl
        self.n_slots = wl.B if n_slots is None else n_slots
        W = wl.cfg.window if window is None else window
        self.desc = stq.make_desc(self.n_slots, wl.H, wl.dk, wl.dv, np.asarray(wl.bits).reshape(-1),
                                  wl.row_weight, wl.cfg.gate, wl.cfg.unit, W, n_comp)
        nbytes = stq.stq_pool_bytes(self.desc)
        self.buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        self.pool = stq.stq_pool_create(self.desc, self.buf)
        self.ref = orc.OraclePool(self.n_slots, wl.H, wl.dk, wl.dv, np.asarray(wl.bits).reshape(-1),
                                  wl.row_weight, wl.cfg.gate, wl.cfg.unit, W, n_comp=n_comp)
        assert self.ref.nbytes == nbytes

    def image(self):
        import torch
        torch.cuda.synchronize()
        return self.buf.cpu().numpy()

    def slots_t(self, slots):
        import torch
        return torch.as_tensor(np.asarray(slots, np.int32), device="cuda")

    def store(self, slots, S):
        import torch
        self.stq.stq_pool_store(self.pool, self.slots_t(slots), torch.as_tensor(S, device="cuda"))
        self.ref.store(slots, S)

    def gpu_step(self, slots, q, k, v, a, b):
        import torch
        dev = lambda x: torch.as_tensor(x, device="cuda")
        o = torch.empty((len(slots), self.wl.H, self.wl.dv), dtype=torch.float32, device="cuda")
        self.stq.stq_decode_step(self.pool, self.slots_t(slots), dev(q), dev(k), dev(v), dev(a), dev(b), o)
        torch.cuda.synchronize()
        return o.cpu().numpy()


def _bf16(bits):
    return (np.asarray(bits, np.uint32) << 16).view(np.float32).astype(np.float64)


def scale_mismatches(sg, cg, sr, cr, code_diff, quant_rows):
    """Row and column scales of one tile compared as the dequantisation steps
    they define: the stored pair (sigma, c) is (s 2^-E, t 2^E), and a different
    E moves every sigma and c by one power of two without changing any step
    sigma_i c_j, so the common factor is divided out first.  Returns (number
    of row or column scales that differ, number of those with no differing
    code in their row or column, largest distance in bf16 steps).  A scale one
    bf16 step off need not move any code of a narrow row (a 4-bit code moves
    by at most 7/128 of a step), so the second count is a report, not a bar.
    code_diff: [d_k][d_v] bool over the rows of quant_rows (binary16 pivot
    rows carry no scales)."""
    qs, rs = _bf16(sg)[quant_rows], _bf16(sr)[quant_rows]
    if qs.size == 0:
        return 0, 0, 0
    ratio = qs / rs
    k = 0
    if np.all(ratio > 0):
        lr = np.log2(ratio)
        ints = lr[lr == np.round(lr)]
        if ints.size:
            vals, cnt = np.unique(ints, return_counts=True)
            k = int(vals[np.argmax(cnt)])
    row_bad = qs != rs * 2.0 ** k
    col_bad = _bf16(cg) != _bf16(cr) * 2.0 ** -k
    rows_with = code_diff.any(axis=1)
    cols_with = code_diff.any(axis=0)
    n = int(row_bad.sum() + col_bad.sum())
    unexplained = int((row_bad & ~rows_with).sum() + (col_bad & ~cols_with).sum())
    # positive bf16 values order like their bit patterns; 2^k adds 128 k to them
    dr = np.abs(np.asarray(sg, np.int64)[quant_rows] - (np.asarray(sr, np.int64)[quant_rows] + 128 * k))
    dc = np.abs(np.asarray(cg, np.int64) - (np.asarray(cr, np.int64) - 128 * k))
    steps = int(max(dr[row_bad].max(initial=0), dc[col_bad].max(initial=0)))
    return n, unexplained, steps


def compare_codes(orc, ref_pool, img_gpu, img_ref, slots, heads=None):
    """Code and scale agreement between two pool images over the given tiles.
    Returns dict with code mismatch count/total, max |dQ|, scale mismatches
    (after the common power of two of each tile) and how many of those have
    no code mismatch in their row or column, pivot mismatches."""
    H = ref_pool.H
    heads = range(H) if heads is None else heads
    res = dict(codes=0, mism=0, maxd=0, scales=0, scale_mism=0, scale_unexpl=0, scale_steps=0, piv=0, piv_bad=0,
               piv_mism=0)
    for s in slots:
        for h in heads:
            Qg, sg, cg, nb = ref_pool.decode_tile(int(s), h, img_gpu)
            Qr, sr, cr, _ = ref_pool.decode_tile(int(s), h, img_ref)
            piv = nb == 16
            if piv.any():
                fg = Qg[piv].astype(np.uint16).view(np.float16).astype(np.float64)
                fr = Qr[piv].astype(np.uint16).view(np.float16).astype(np.float64)
                res["piv"] += fg.size
                res["piv_mism"] += int(np.count_nonzero(fg != fr))
                # a mismatch must be one binary16 rounding step of the value, or lie
                # within binary32 cancellation noise of the row (S' = aH + k delta)
                step = np.maximum(np.abs(fr), np.abs(fg)) * 2.0 ** -10 + 2.0 ** -24
                floor = 2.0 ** -20 * np.abs(fr).max(axis=1, keepdims=True)
                res["piv_bad"] += int(np.sum(np.abs(fg - fr) > np.maximum(step, floor)))
            if (~piv).any():
                d = np.abs(Qg[~piv] - Qr[~piv])
                res["codes"] += d.size
                res["mism"] += int(np.count_nonzero(d))
                res["maxd"] = max(res["maxd"], int(d.max()))
                quant_rows = ~piv
                qd = (Qg != Qr) & quant_rows[:, None]
                res["scales"] += int(quant_rows.sum()) + cg.size
                n, un, st = scale_mismatches(sg, cg, sr, cr, qd[quant_rows], quant_rows)
                res["scale_mism"] += n
                res["scale_unexpl"] += un
                res["scale_steps"] = max(res["scale_steps"], st)
    return res


def readout_ok(o_gpu, o_ref, tol=1e-3):
    """Per tile: |o - o_ref| <= tol * (|o_ref| + 0.01 * max|o_ref|) elementwise."""
    o_ref = o_ref.astype(np.float64)
    scale = np.abs(o_ref).max(axis=-1, keepdims=True)
    err = np.abs(o_gpu.astype(np.float64) - o_ref)
    bound = tol * (np.abs(o_ref) + 0.01 * scale) + 1e-30
    return float((err / bound).max())


AGG_SUM = ("mism", "codes", "scale_mism", "scale_unexpl", "scales", "piv_bad", "piv", "piv_mism")


def new_agg():
    """Running totals of compare_codes results over several steps or tiles."""
    d = {k: 0 for k in AGG_SUM}
    d.update(maxd=0, scale_steps=0, o=0.0)
    return d


def add_agg(agg, r, o=None):
    for k in AGG_SUM:
        agg[k] += r[k]
    agg["maxd"] = max(agg["maxd"], r["maxd"])
    agg["scale_steps"] = max(agg["scale_steps"], r["scale_steps"])
    if o is not None:
        agg["o"] = max(agg["o"], o)
    return agg


def agg_text(r):
    return ("code mismatch %d of %d (%.1e, max |dQ| %d), scale mismatch %d of %d (max %d bf16 steps; %d with "
            "no differing code in their row or column), pivot mismatch %d of %d (beyond one step %d)"
            % (r["mism"], r["codes"], r["mism"] / max(r["codes"], 1), r["maxd"], r["scale_mism"], r["scales"],
               r["scale_steps"], r["scale_unexpl"], r["piv_mism"], r["piv"], r["piv_bad"]))
