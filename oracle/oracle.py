"""numpy/ctypes front end of the C oracle (test infrastructure only)."""
import ctypes
import os
import subprocess

import numpy as np

_DIR = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_DIR, "stq_oracle.c")
_LIB = os.path.join(_DIR, "libstq_oracle.so")
_CFLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fexcess-precision=standard",
           "-fno-fast-math", "-fPIC", "-shared", "-Wall"]

__all__ = ["build", "lib", "refit", "dequant", "requant_fixed", "pack", "unpack",
           "tile_bytes", "tile_stride", "update_f64", "pack_rows", "unpack_rows", "row_tile_bytes", "OraclePool", "num_threads", "set_num_threads", "clip_events"]


def build(force=False):
    """Compile the oracle with gcc (binary32 ops, no contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc"] + _CFLAGS + ["-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        # STQ_ORACLE_LIB: a copy of the oracle compiled elsewhere (the planted-
        # mistake tests load mutated copies this way); otherwise this one
        path = os.environ.get("STQ_ORACLE_LIB")
        if not path:
            build()
            path = _LIB
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        I = ctypes.c_int
        L.orc_tile_bytes.restype = ctypes.c_size_t
        L.orc_tile_bytes.argtypes = [I, I, I]
        L.orc_tile_stride.restype = ctypes.c_size_t
        L.orc_tile_stride.argtypes = [I, I, I]
        L.orc_refit.argtypes = [I, I, P, P, P, P, P, P, P]
        L.orc_dequant.argtypes = [I, I, P, P, P, P, P]
        L.orc_requant_fixed.argtypes = [I, I, P, P, P, P, P]
        L.orc_pack.argtypes = [I, I, I, P, P, P, P]
        L.orc_unpack.argtypes = [I, I, I, P, P, P, P]
        L.orc_pack_rows.argtypes = [I, I, P, P, P, P, P]
        L.orc_unpack_rows.argtypes = [I, I, P, P, P, P, P]
        D = [I, I, I, I, I, I, I, P]
        L.orc_pool_bytes.restype = ctypes.c_size_t
        L.orc_pool_bytes.argtypes = D
        L.orc_pool_init.argtypes = D + [P, P]
        L.orc_pool_store.argtypes = D + [P, P, I, P]
        L.orc_pool_fetch.argtypes = D + [P, P, I, P]
        L.orc_pool_requant_fixed.argtypes = D + [P, P, I]
        L.orc_decode_step.argtypes = D + [P, P, I, P, P, P, P, P, P]
        L.orc_window_flush.argtypes = D + [P, P, I]
        L.orc_prefill.argtypes = D + [P, P, I, P, P, P, P, P, P, P, P]
        L.orc_update_f64.argtypes = [I, I, P, P, P, P, P, I, ctypes.c_double, P, P]
        L.orc_num_threads.restype = I
        L.orc_set_threads.argtypes = [I]
        L.orc_clip_events.restype = ctypes.c_long
        _lib = L
    return _lib


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


def num_threads():
    return lib().orc_num_threads()


def set_num_threads(n):
    """Threads of the oracle's parallel loops over tiles (timing only)."""
    lib().orc_set_threads(int(n))


def clip_events():
    return lib().orc_clip_events()


def tile_bytes(n, dk, dv):
    return lib().orc_tile_bytes(n, dk, dv)


def tile_stride(n, dk, dv):
    return lib().orc_tile_stride(n, dk, dv)


def refit(S, w, nb):
    """R on one fp32 tile.  nb: width per row (16 = pivot).
    Returns (sigma bf16 bits, c bf16 bits, Q int32 (pivot rows: binary16 bits), E)."""
    S = _c(S, np.float32)
    dk, dv = S.shape
    w = _c(w, np.float32)
    nb = _c(np.broadcast_to(nb, (dk,)), np.int32)
    sig = np.zeros(dk, np.uint16)
    cst = np.zeros(dv, np.uint16)
    Q = np.zeros((dk, dv), np.int32)
    E = np.zeros(1, np.int32)
    lib().orc_refit(dk, dv, _p(S), _p(w), _p(nb), _p(sig), _p(cst), _p(Q), _p(E))
    return sig, cst, Q, int(E[0])


def update_f64(S, q, k, v, a, b):
    """Binary64 gated delta update + readout of one tile.  a: scalar (GDN) or
    [dk] (KDA).  Returns (S', o)."""
    S = _c(S, np.float64)
    dk, dv = S.shape
    a = np.atleast_1d(_c(a, np.float64))
    per_row = 1 if a.size == dk and dk > 1 else 0
    Sp = np.zeros((dk, dv), np.float64)
    o = np.zeros(dv, np.float64)
    lib().orc_update_f64(dk, dv, _p(S), _p(_c(q, np.float64)), _p(_c(k, np.float64)),
                         _p(_c(v, np.float64)), _p(a), per_row, float(b), _p(Sp), _p(o))
    return Sp, o


def dequant(sig, cst, Q, nb):
    Q = _c(Q, np.int32)
    dk, dv = Q.shape
    nb = _c(np.broadcast_to(nb, (dk,)), np.int32)
    S = np.zeros((dk, dv), np.float32)
    lib().orc_dequant(dk, dv, _p(_c(sig, np.uint16)), _p(_c(cst, np.uint16)), _p(Q), _p(nb), _p(S))
    return S


def requant_fixed(S, sig, cst, nb):
    S = _c(S, np.float32)
    dk, dv = S.shape
    nb = _c(np.broadcast_to(nb, (dk,)), np.int32)
    Q = np.zeros((dk, dv), np.int32)
    lib().orc_requant_fixed(dk, dv, _p(S), _p(_c(sig, np.uint16)), _p(_c(cst, np.uint16)), _p(nb), _p(Q))
    return Q


def pack(n, Q, sig, cst):
    Q = _c(Q, np.int32)
    dk, dv = Q.shape
    t = np.zeros(tile_bytes(n, dk, dv), np.uint8)
    lib().orc_pack(n, dk, dv, _p(Q), _p(_c(sig, np.uint16)), _p(_c(cst, np.uint16)), _p(t))
    return t


def row_tile_bytes(nb, dv):
    return int(sum(dv * int(n) // 8 for n in nb)) + 2 * (len(nb) + dv)


def pack_rows(nb, Q, sig, cst):
    """Row-record tile of a per-row-width head (rows sorted by width)."""
    Q = _c(Q, np.int32)
    dk, dv = Q.shape
    nb = _c(nb, np.int32)
    t = np.zeros(row_tile_bytes(nb, dv), np.uint8)
    lib().orc_pack_rows(dk, dv, _p(nb), _p(Q), _p(_c(sig, np.uint16)), _p(_c(cst, np.uint16)), _p(t))
    return t


def unpack_rows(nb, dv, tile):
    nb = _c(nb, np.int32)
    dk = nb.size
    tile = _c(tile, np.uint8)
    Q = np.zeros((dk, dv), np.int32)
    sig = np.zeros(dk, np.uint16)
    cst = np.zeros(dv, np.uint16)
    lib().orc_unpack_rows(dk, dv, _p(nb), _p(tile), _p(Q), _p(sig), _p(cst))
    return Q, sig, cst


def unpack(n, dk, dv, tile):
    tile = _c(tile, np.uint8)
    Q = np.zeros((dk, dv), np.int32)
    sig = np.zeros(dk, np.uint16)
    cst = np.zeros(dv, np.uint16)
    lib().orc_unpack(n, dk, dv, _p(tile), _p(Q), _p(sig), _p(cst))
    return Q, sig, cst


class OraclePool:
    """Host image of a whole pool buffer, advanced by the oracle."""

    def __init__(self, n_slots, n_heads, d_k, d_v, bits, row_weight, gate_kind=0,
                 unit_kind=0, window=0, image=None, n_comp=0):
        self.n_slots, self.H, self.dk, self.dv = n_slots, n_heads, d_k, d_v
        self.gate, self.unit, self.W, self.C = gate_kind, unit_kind, window, n_comp
        self.bits = _c(bits, np.int32)
        self.wt = _c(row_weight, np.float32).reshape(n_heads, d_k)
        self.nbytes = lib().orc_pool_bytes(*self._d())
        if image is None:
            self.img = np.zeros(self.nbytes, np.uint8)
            lib().orc_pool_init(*self._d(), _p(self.wt), _p(self.img))
        else:
            assert image.size == self.nbytes
            self.img = _c(image, np.uint8).copy()

    def _d(self):
        # the window argument carries the compensator count in its high half
        return (self.n_slots, self.H, self.dk, self.dv, self.gate, self.unit, self.W | (self.C << 16),
                _p(self.bits))

    def store(self, slots, S):
        slots = _c(slots, np.int32)
        S = _c(S, np.float32)
        assert S.shape == (slots.size, self.H, self.dk, self.dv)
        lib().orc_pool_store(*self._d(), _p(self.img), _p(slots), slots.size, _p(S))

    def fetch(self, slots):
        slots = _c(slots, np.int32)
        S = np.zeros((slots.size, self.H, self.dk, self.dv), np.float32)
        lib().orc_pool_fetch(*self._d(), _p(self.img), _p(slots), slots.size, _p(S))
        return S

    def requant_fixed(self, slots):
        slots = _c(slots, np.int32)
        lib().orc_pool_requant_fixed(*self._d(), _p(self.img), _p(slots), slots.size)

    def step(self, slots, q, k, v, a, b):
        """One decode token; returns the binary64 readout o [n][H][d_v]."""
        slots = _c(slots, np.int32)
        n = slots.size
        q = _c(q, np.float32).reshape(n, self.H, self.dk)
        k = _c(k, np.float32).reshape(n, self.H, self.dk)
        v = _c(v, np.float32).reshape(n, self.H, self.dv)
        a = _c(a, np.float32)
        assert a.size == (n * self.H * self.dk if self.gate else n * self.H)
        b = _c(b, np.float32).reshape(n, self.H)
        o = np.zeros((n, self.H, self.dv), np.float64)
        lib().orc_decode_step(*self._d(), _p(self.img), _p(slots), n, _p(q), _p(k), _p(v),
                              _p(a), _p(b), _p(o))
        return o

    def prefill(self, slots, seq_start, q, k, v, a, b, final_state=False):
        """Prefill ingest of token-major sequences (request c owns tokens
        seq_start[c] .. seq_start[c+1]-1); returns the binary64 readouts
        o [tok][H][d_v] and, if asked, the binary64 final states [n][H][d_k][d_v]."""
        slots = _c(slots, np.int32)
        n = slots.size
        ss = _c(seq_start, np.int32)
        assert ss.size == n + 1 and np.all(np.diff(ss) >= 0) and ss[0] >= 0
        T = int(ss[-1])
        q = _c(q, np.float32).reshape(T, self.H, self.dk)
        k = _c(k, np.float32).reshape(T, self.H, self.dk)
        v = _c(v, np.float32).reshape(T, self.H, self.dv)
        a = _c(a, np.float32)
        assert a.size == (T * self.H * self.dk if self.gate else T * self.H)
        b = _c(b, np.float32).reshape(T, self.H)
        o = np.zeros((T, self.H, self.dv), np.float64)
        Sf = np.zeros((n, self.H, self.dk, self.dv), np.float64) if final_state else None
        lib().orc_prefill(*self._d(), _p(self.img), _p(slots), n, _p(ss), _p(q), _p(k), _p(v),
                          _p(a), _p(b), _p(o), _p(Sf) if final_state else None)
        return (o, Sf) if final_state else o

    def window_flush(self, slots):
        slots = _c(slots, np.int32)
        lib().orc_window_flush(*self._d(), _p(self.img), _p(slots), slots.size)

    # byte views ------------------------------------------------------
    def hdr_bytes(self):
        ru = lambda x: (x + 255) // 256 * 256
        roff = ru(ru(64 + 8 * self.H) + 4 * self.H * self.dk)
        if self.unit == 1:
            return ru(roff + 2 * self.H * self.dk + 16 * self.H)
        return roff

    def head_bits(self, h):
        """Width of every row of head h."""
        if self.unit == 1:
            return self.bits.reshape(self.H, self.dk)[h]
        return np.full(self.dk, int(self.bits[h]), np.int32)

    def _tile_bytes(self, h):
        if self.unit == 1:
            return row_tile_bytes(self.head_bits(h), self.dv)
        return tile_bytes(int(self.bits[h]), self.dk, self.dv)

    def head_offsets(self):
        offs, s = [], 0
        for h in range(self.H):
            offs.append(s)
            s += (self._tile_bytes(h) + 255) // 256 * 256
        return offs, s

    def tile_view(self, slot, h, img=None):
        img = self.img if img is None else img
        offs, sb = self.head_offsets()
        base = self.hdr_bytes() + slot * sb + offs[h]
        return img[base: base + self._tile_bytes(h)]

    def cache_stride(self):
        return 256 + 4 * self.W * (self.dk + self.dv) + 4 * self.C * self.dv if self.W else 0

    def cache_view(self, slot, h, img=None):
        """(count, G[W], K[W][dk], U[W][dv], comp rows[C], comp values[C][dv]) of a tile's window."""
        img = self.img if img is None else img
        _, sb = self.head_offsets()
        st = self.cache_stride()
        base = self.hdr_bytes() + self.n_slots * sb + (slot * self.H + h) * st
        c = img[base: base + st]
        W, dk, dv = self.W, self.dk, self.dv
        kend = 256 + 4 * W * dk
        uend = kend + 4 * W * dv
        return (int(c[0:4].view(np.int32)[0]), c[4: 4 + 4 * W].view(np.float32),
                c[256:kend].view(np.float32).reshape(W, dk), c[kend:uend].view(np.float32).reshape(W, dv),
                c[192: 192 + 4 * self.C].view(np.int32), c[uend:].view(np.float32).reshape(self.C, dv))

    def decode_tile(self, slot, h, img=None):
        """(Q, sigma, c, widths) of one tile, rows in original order."""
        t = self.tile_view(slot, h, img)
        nb = self.head_bits(h)
        if self.unit == 1:
            Q, sg, cs = unpack_rows(nb, self.dv, t)
        else:
            Q, sg, cs = unpack(int(self.bits[h]), self.dk, self.dv, t)
        return Q, sg, cs, nb
