"""Seeded synthetic workloads for the decode step (inputs only).

This module draws random inputs with the shapes, distributions and structure
the pages describe; it holds none of the method's arithmetic and is shared by
the tests, the oracle runs and the benchmark.  Every draw is seeded
(numpy PCG64); the initial state of a slot depends only on (seed, slot) so a
sample of slots can be regenerated alone.

Structure taken from the pages (cited by page title and section):
 - head dimension 128 and 16-bit scales per row/column: gpt-diffusion
   STEPQuant analysis, "Qué dice realmente el «6-bit»";
 - row and column outliers that persist during decoding, row impact spread of
   about two orders of magnitude: STEPQuant talk preview (qingkeai.online),
   "高并发场景下的显存困境…"; e-cogni analysis, "Como funciona";
 - heavy-tailed lifetimes (gate half-lives): talk preview, same section;
   gpt-diffusion analysis, "Las dos ideas";
 - bit units = head (GDN) or key row (KDA), FP16 pivots for the hardest units:
   gpt-diffusion analysis, "Las dos ideas".
"""
from dataclasses import dataclass, field

import numpy as np

GATE_HEAD, GATE_CHANNEL = 0, 1
UNIT_HEAD, UNIT_ROW = 0, 1


@dataclass
class Config:
    key: str
    workload: str
    B: int
    H: int
    dk: int
    dv: int
    T: int
    gate: int
    unit: int
    window: int
    seed: int
    bits: str              # "uniform8", "uniform4", "gdn_mix", "kda_rows"
    weights: str           # "uniform_0.5_2", "lognormal", "ones"
    state: str             # "plain", "profiled"
    gate_law: str          # "softplus", "gdn_halflife", "kda_halflife"
    persistent_io: bool = False
    extra: dict = field(default_factory=dict)


CONFIGS = {
    "C1": Config("C1", "tiny uniform 8-bit, B=4 H=2 d=64 T=32", 4, 2, 64, 64, 32,
                 GATE_HEAD, UNIT_HEAD, 0, 1001, "uniform8", "uniform_0.5_2", "plain", "softplus"),
    "C2": Config("C2", "GDN one step, B=64 H=32 d=128, 6-bit nominal mix", 64, 32, 128, 128, 1,
                 GATE_HEAD, UNIT_HEAD, 0, 1002, "gdn_mix", "lognormal", "profiled", "gdn_halflife"),
    "C3": Config("C3", "GDN serving pool, B=512 H=32 d=128, 6-bit nominal mix, 64 steps", 512, 32,
                 128, 128, 64, GATE_HEAD, UNIT_HEAD, 0, 1003, "gdn_mix", "lognormal", "profiled",
                 "gdn_halflife", persistent_io=True),
    "C4": Config("C4", "KDA per-channel gate, B=256 H=32 d=128, per-row bits, 32 steps", 256, 32,
                 128, 128, 32, GATE_CHANNEL, UNIT_ROW, 0, 1004, "kda_rows", "lognormal",
                 "profiled", "kda_halflife", persistent_io=True),
    "C5": Config("C5", "windowed 4-bit GDN, B=512 H=32 d=128, W=16, 64 steps", 512, 32, 128, 128,
                 64, GATE_HEAD, UNIT_HEAD, 16, 1005, "uniform4", "ones", "profiled",
                 "gdn_halflife", persistent_io=True),
}


def quotas(fracs, total):
    """Largest-remainder integer quotas of `total` units for the given fractions."""
    raw = np.asarray(fracs, np.float64) * total
    q = np.floor(raw).astype(np.int64)
    rem = total - int(q.sum())
    order = np.argsort(-(raw - q), kind="stable")
    q[order[:rem]] += 1
    return q


class Workload:
    """Inputs of one configuration, optionally with fewer requests (B)."""

    def __init__(self, key, B=None, T=None, H=None):
        c = CONFIGS[key]
        self.cfg = c
        self.B = c.B if B is None else B
        self.T = c.T if T is None else T
        self.H = c.H if H is None else H
        self.dk, self.dv = c.dk, c.dv
        self.seed = c.seed
        self._plan()

    # -- static plan: bit map, row weights, head profiles, lifetimes ------
    def _rng(self, *tag):
        return np.random.default_rng([self.seed] + list(tag))

    def _plan(self):
        c, H, dk, dv = self.cfg, self.H, self.dk, self.dv
        g = self._rng(0)
        if c.bits == "uniform8":
            self.bits = np.full(H, 8, np.int32)
        elif c.bits == "uniform4":
            self.bits = np.full(H, 4, np.int32)
        elif c.bits == "gdn_mix":
            q = quotas([0.30, 0.50, 0.18, 0.02], H)
            b = np.repeat(np.array([4, 6, 8, 16], np.int32), q)
            self.bits = g.permutation(b).astype(np.int32)
        elif c.bits == "kda_rows":
            q = quotas([0.30, 0.50, 0.19, 0.01], H * dk)
            b = np.repeat(np.array([4, 6, 8, 16], np.int32), q)
            self.bits = g.permutation(b).astype(np.int32).reshape(H, dk)
        else:
            raise ValueError(c.bits)
        g = self._rng(1)
        if c.weights == "uniform_0.5_2":
            self.row_weight = g.uniform(0.5, 2.0, (H, dk)).astype(np.float32)
        elif c.weights == "lognormal":
            self.row_weight = np.clip(np.exp(g.normal(0.0, 1.15, (H, dk))), 0.1, 10.0).astype(np.float32)
        else:
            self.row_weight = np.ones((H, dk), np.float32)
        # per-head row/column magnitude profiles with persistent outliers
        g = self._rng(2)
        self.r_prof = np.empty((H, dk))
        self.c_prof = np.empty((H, dv))
        for h in range(H):
            if c.state == "plain":
                r = np.ones(dk)
                cc = np.ones(dv)
            else:
                r = np.exp(g.normal(0.0, 1.5, dk))
                cc = np.exp(g.normal(0.0, 1.5, dv))
            orow = g.choice(dk, 2, replace=False)
            ocol = g.choice(dv, 1)
            r[orow] *= 20.0
            cc[ocol] *= 10.0
            self.r_prof[h], self.c_prof[h] = r, cc
        # gate lifetimes
        g = self._rng(3)
        if c.gate_law == "gdn_halflife":
            u = g.uniform(0.0, 1.0, H)
            u = np.maximum(u, 1e-12)
            self.half_life = np.clip(6.58 / u, 6.58, 6931.0)
        elif c.gate_law == "kda_halflife":
            self.half_life = 10.0 ** g.uniform(0.0, 4.0, (H, dk))
        else:
            self.half_life = None

    # -- initial state -------------------------------------------------------
    def state(self, slots):
        """S0 fp32 [len(slots)][H][dk][dv]; slot s depends only on (seed, s)."""
        slots = np.asarray(slots, np.int64).reshape(-1)
        out = np.empty((slots.size, self.H, self.dk, self.dv), np.float32)
        for n, s in enumerate(slots):
            z = self._rng(4, int(s)).standard_normal((self.H, self.dk, self.dv))
            out[n] = 0.1 * z * self.r_prof[:, :, None] * self.c_prof[:, None, :]
        return out

    # -- per-token inputs ---------------------------------------------------
    def token(self, t, n=None):
        """(q, k, v, a, b) for token t and the first n requests (default B)."""
        n = self.B if n is None else n
        return self._io(self._rng(5, int(t)), n)

    def _io(self, g, n):
        """One draw of (q, k, v, a, b) with leading axis n, in a fixed order."""
        H, dk, dv = self.H, self.dk, self.dv
        q = g.standard_normal((n, H, dk))
        k = g.standard_normal((n, H, dk))
        v = g.standard_normal((n, H, dv))
        if self.cfg.persistent_io:
            rbar = self.r_prof / np.exp(np.log(self.r_prof).mean(axis=1, keepdims=True))
            cbar = self.c_prof / np.exp(np.log(self.c_prof).mean(axis=1, keepdims=True))
            k = k * np.sqrt(rbar)[None]
            v = v * cbar[None]
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
        b = g.uniform(0.05, 0.95, (n, H))
        law = self.cfg.gate_law
        if law == "softplus":
            x = g.normal(-3.0, 1.0, (n, H))
            a = np.exp(-np.logaddexp(0.0, x))
        elif law == "gdn_halflife":
            hp = self.half_life[None, :] * np.exp(0.1 * g.standard_normal((n, H)))
            a = np.clip(2.0 ** (-1.0 / hp), 0.9, 0.9999)
        else:
            hp = self.half_life[None] * np.exp(0.1 * g.standard_normal((n, H, dk)))
            a = 2.0 ** (-1.0 / hp)
        f = np.float32
        return q.astype(f), k.astype(f), v.astype(f), a.astype(f), b.astype(f)

    def prompts(self, lens):
        """Token-major prompt inputs for requests of the given lengths:
        (seq_start [n+1] int32, q, k, v [tok][H][d], a, b [tok][H] (per-channel
        gate: a [tok][H][dk])); request c's tokens are drawn with the per-token
        law from a stream that depends only on (seed, c)."""
        lens = [int(x) for x in lens]
        ss = np.zeros(len(lens) + 1, np.int32)
        ss[1:] = np.cumsum(lens)
        parts = [self._io(self._rng(6, c), L) for c, L in enumerate(lens)]
        cat = [np.concatenate([p[i] for p in parts], axis=0) for i in range(5)]
        return (ss,) + tuple(cat)
