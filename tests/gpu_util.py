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


def compare_codes(orc, ref_pool, img_gpu, img_ref, slots, heads=None):
    """Code and scale agreement between two pool images over the given tiles.
    Returns dict with code mismatch count/total, max |dQ|, scale mismatches,
    pivot max relative error."""
    H = ref_pool.H
    heads = range(H) if heads is None else heads
    res = dict(codes=0, mism=0, maxd=0, scales=0, scale_mism=0, piv=0, piv_bad=0, piv_mism=0)
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
                res["scales"] += sg.size + cg.size
                res["scale_mism"] += int(np.count_nonzero(sg != sr) + np.count_nonzero(cg != cr))
    return res


def readout_ok(o_gpu, o_ref, tol=1e-3):
    """Per tile: |o - o_ref| <= tol * (|o_ref| + 0.01 * max|o_ref|) elementwise."""
    o_ref = o_ref.astype(np.float64)
    scale = np.abs(o_ref).max(axis=-1, keepdims=True)
    err = np.abs(o_gpu.astype(np.float64) - o_ref)
    bound = tol * (np.abs(o_ref) + 0.01 * scale) + 1e-30
    return float((err / bound).max())
