"""ctypes marshalling for libstq.so (no computation happens here)."""
import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
_PATH = os.path.join(_PKG, "libstq.so")

STQ_OK = 0
STQ_GATE_HEAD, STQ_GATE_CHANNEL = 0, 1
STQ_UNIT_HEAD, STQ_UNIT_ROW = 0, 1


class StqError(RuntimeError):
    def __init__(self, status, what):
        super().__init__("%s: %s" % (what, stq_status_str(status)))
        self.status = status


class _Desc(ctypes.Structure):
    _fields_ = [("n_slots", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("gate_kind", ctypes.c_int32), ("unit_kind", ctypes.c_int32),
                ("window", ctypes.c_int32), ("n_comp", ctypes.c_int32),
                ("unit_bits", ctypes.POINTER(ctypes.c_int32)),
                ("row_weight", ctypes.POINTER(ctypes.c_float))]


def library_path():
    return _PATH


def _load():
    if not os.path.exists(_PATH):
        raise ImportError("libstq.so is not built (%s); run quantized_linear_attention_amd/build.py "
                          "or __graft_entry__.build()" % _PATH)
    L = ctypes.CDLL(_PATH)
    P, I, St = ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p
    DP = ctypes.POINTER(_Desc)
    L.stq_status_str.restype = ctypes.c_char_p
    L.stq_status_str.argtypes = [I]
    L.stq_pool_bytes.restype = ctypes.c_size_t
    L.stq_pool_bytes.argtypes = [DP]
    L.stq_pool_create.restype = I
    L.stq_pool_create.argtypes = [DP, P, ctypes.c_size_t, St, ctypes.POINTER(P)]
    L.stq_pool_destroy.restype = I
    L.stq_pool_destroy.argtypes = [P]
    for name in ("stq_pool_store", "stq_pool_fetch"):
        getattr(L, name).restype = I
        getattr(L, name).argtypes = [P, P, I, P, St]
    L.stq_decode_step.restype = I
    L.stq_decode_step.argtypes = [P, P, I, P, P, P, P, P, P, St]
    L.stq_prefill.restype = I
    L.stq_prefill_states.restype = I
    L.stq_prefill_states.argtypes = [I, I, I, I, I, P, P, P, P, P, P, P, P, St]
    L.stq_decode_readout.restype = I
    L.stq_decode_readout.argtypes = [P, P, I, P, P, P, P, P, P, St]
    L.stq_decode_commit.restype = I
    L.stq_decode_commit.argtypes = [P, P, I, P, P, P, P, P, St]
    L.stq_allocate_bits.restype = I
    L.stq_allocate_bits.argtypes = [I, P, P, I, ctypes.c_double, P, P]
    L.stq_prefill.argtypes = [P, P, I, P, P, P, P, P, P, P, St]
    for name in ("stq_window_flush", "stq_requant_fixed_scales"):
        getattr(L, name).restype = I
        getattr(L, name).argtypes = [P, P, I, St]
    return L


_L = _load()


def stq_status_str(status):
    return _L.stq_status_str(int(status)).decode()


def _check(status, what):
    if status != STQ_OK:
        raise StqError(status, what)


def make_desc(n_slots, n_heads, d_k, d_v, unit_bits, row_weight, gate_kind=STQ_GATE_HEAD,
              unit_kind=STQ_UNIT_HEAD, window=0, n_comp=0):
    """Build a stq_pool_desc; the returned object keeps its host arrays alive."""
    bits = np.ascontiguousarray(unit_bits, dtype=np.int32).reshape(-1)
    wt = np.ascontiguousarray(row_weight, dtype=np.float32).reshape(-1)
    d = _Desc(int(n_slots), int(n_heads), int(d_k), int(d_v), int(gate_kind), int(unit_kind),
              int(window), int(n_comp), bits.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
              wt.ctypes.data_as(ctypes.POINTER(ctypes.c_float)))
    d._keep = (bits, wt)
    return d


def _stream(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(getattr(stream, "cuda_stream", stream))


def _dev(t, dtype, what, numel=None, device=None):
    """Device pointer of a contiguous CUDA tensor of `dtype`; with `numel`
    and `device`, also checks its element count and device, so that no kernel
    is handed a buffer shorter than the sizes it indexes."""
    if t is None:
        return None
    if not (t.is_cuda and t.is_contiguous() and t.dtype == dtype):
        raise StqError(-1, "%s must be a contiguous %s CUDA tensor" % (what, dtype))
    if numel is not None and t.numel() != numel:
        raise StqError(-1, "%s has %d elements, expected %d" % (what, t.numel(), numel))
    if device is not None and t.device != device:
        raise StqError(-1, "%s is on %s, the pool buffer on %s" % (what, t.device, device))
    return ctypes.c_void_p(t.data_ptr())


def stq_pool_bytes(desc):
    return int(_L.stq_pool_bytes(ctypes.byref(desc)))


class _Pool:
    def __init__(self, handle, desc, buf):
        self.handle, self.desc, self.buf = handle, desc, buf
        self.H, self.dk, self.dv = int(desc.n_heads), int(desc.d_k), int(desc.d_v)
        self.gate, self.unit = int(desc.gate_kind), int(desc.unit_kind)
        self.device = buf.device

    def sizes(self, n):
        """Element counts of the per-token tensors of a call on n requests."""
        H, dk, dv = self.H, self.dk, self.dv
        return {"q": n * H * dk, "k": n * H * dk, "v": n * H * dv, "o": n * H * dv,
                "a": n * H * (dk if self.gate == STQ_GATE_CHANNEL else 1), "b": n * H,
                "S": n * H * dk * dv}

    def __del__(self):
        if getattr(self, "handle", None):
            _L.stq_pool_destroy(self.handle)
            self.handle = None


def stq_pool_create(desc, buf, stream=None):
    """buf: uint8 CUDA tensor of at least stq_pool_bytes(desc) bytes (256-aligned)."""
    import torch
    out = ctypes.c_void_p()
    p = _dev(buf, torch.uint8, "pool buffer")
    _check(_L.stq_pool_create(ctypes.byref(desc), p, buf.numel(), _stream(stream), ctypes.byref(out)),
           "stq_pool_create")
    return _Pool(out, desc, buf)


def stq_pool_destroy(pool):
    if pool.handle:
        _check(_L.stq_pool_destroy(pool.handle), "stq_pool_destroy")
        pool.handle = None


def _slots(slots, pool=None):
    import torch
    return _dev(slots, torch.int32, "slots", device=None if pool is None else pool.device), int(slots.numel())


def _token_args(pool, n, names, tensors):
    """Pointers of the per-token tensors of a call on n requests (or n tokens),
    each checked against the pool's sizes and device."""
    import torch
    want = pool.sizes(n)
    return [_dev(t, torch.float32, nm, want[nm], pool.device) for nm, t in zip(names, tensors)]


def stq_pool_store(pool, slots, S, stream=None):
    """S: fp32 [n][H][d_k][d_v] on the pool's device."""
    sp, n = _slots(slots, pool)
    _check(_L.stq_pool_store(pool.handle, sp, n, _token_args(pool, n, ["S"], [S])[0], _stream(stream)),
           "stq_pool_store")


def stq_pool_fetch(pool, slots, S_out, stream=None):
    sp, n = _slots(slots, pool)
    _check(_L.stq_pool_fetch(pool.handle, sp, n, _token_args(pool, n, ["S"], [S_out])[0], _stream(stream)),
           "stq_pool_fetch")


def stq_decode_step(pool, slots, q, k, v, a, b, o, stream=None):
    sp, n = _slots(slots, pool)
    ptrs = _token_args(pool, n, "qkvabo", (q, k, v, a, b, o))
    _check(_L.stq_decode_step(pool.handle, sp, n, *ptrs, _stream(stream)), "stq_decode_step")


def _prompt_tokens(pool_or_dims, n, seq_start, q):
    """Token count of a packed prompt batch, from q's size, and the checks that
    need the start offsets: n + 1 entries, the last within the batch.  Reading
    the last offset copies one int32 from the device (a synchronisation of
    the current stream); the prefill is not on the per-token path."""
    import torch
    H, dk = pool_or_dims
    if seq_start is None or seq_start.numel() != n + 1:
        raise StqError(-1, "seq_start must have n + 1 = %d entries" % (n + 1))
    if q is None or q.numel() % (H * dk):
        raise StqError(-1, "q must be [tokens][H][d_k]")
    tok = q.numel() // (H * dk)
    _dev(seq_start, torch.int32, "seq_start", n + 1, q.device)
    last = int(seq_start[-1].item()) if n else 0
    if last > tok:
        raise StqError(-1, "seq_start[n] = %d exceeds the %d tokens of q" % (last, tok))
    return tok


def stq_prefill(pool, slots, seq_start, q, k, v, a, b, o, stream=None):
    import torch
    sp, n = _slots(slots, pool)
    tok = _prompt_tokens((pool.H, pool.dk), n, seq_start, q)
    ptrs = _token_args(pool, tok, "qkvabo", (q, k, v, a, b, o))
    _check(_L.stq_prefill(pool.handle, sp, n, _dev(seq_start, torch.int32, "seq_start"), *ptrs,
                          _stream(stream)),
           "stq_prefill")


def stq_allocate_bits(err, half_life, n_pivots, budget_bits):
    """Host numpy arrays: err [n][3] (4, 6, 8 bits), half_life [n]; returns (bits [n] int32, objective)."""
    import numpy as np
    e = np.ascontiguousarray(err, np.float64)
    hl = np.ascontiguousarray(half_life, np.float64)
    n = hl.size
    if e.shape != (n, 3):
        raise StqError(-1, "err must be [n][3]")
    bits = np.zeros(n, np.int32)
    obj = ctypes.c_double(0.0)
    _check(_L.stq_allocate_bits(n, e.ctypes.data_as(ctypes.c_void_p), hl.ctypes.data_as(ctypes.c_void_p),
                                int(n_pivots), float(budget_bits), bits.ctypes.data_as(ctypes.c_void_p),
                                ctypes.byref(obj)), "stq_allocate_bits")
    return bits, obj.value


class _Dims:
    """Sizes of a plain-state prefill, laid out as a pool's would be."""
    def __init__(self, H, dk, dv, gate, device):
        self.H, self.dk, self.dv, self.gate, self.device = H, dk, dv, gate, device

    sizes = _Pool.sizes


def stq_prefill_states(S, seq_start, q, k, v, a, b, o, gate_kind=STQ_GATE_HEAD, stream=None):
    """S: contiguous fp32 CUDA tensor [n][H][d_k][d_v], advanced in place."""
    import torch
    f = torch.float32
    if S is None or S.dim() != 4:
        raise StqError(-1, "S must be [n][H][d_k][d_v]")
    n, H, dk, dv = S.shape
    Sp = _dev(S, f, "S")
    dims = _Dims(H, dk, dv, int(gate_kind), S.device)
    tok = _prompt_tokens((H, dk), n, seq_start, q)
    ptrs = _token_args(dims, tok, "qkvabo", (q, k, v, a, b, o))
    _check(_L.stq_prefill_states(n, H, dk, dv, gate_kind, Sp, _dev(seq_start, torch.int32, "seq_start"), *ptrs,
                                 _stream(stream)),
           "stq_prefill_states")


def stq_decode_readout(pool, slots, q, k, v, a, b, o, stream=None):
    sp, n = _slots(slots, pool)
    ptrs = _token_args(pool, n, "qkvabo", (q, k, v, a, b, o))
    _check(_L.stq_decode_readout(pool.handle, sp, n, *ptrs, _stream(stream)), "stq_decode_readout")


def stq_decode_commit(pool, slots, q, k, v, a, b, stream=None):
    sp, n = _slots(slots, pool)
    ptrs = _token_args(pool, n, "qkvab", (q, k, v, a, b))
    _check(_L.stq_decode_commit(pool.handle, sp, n, *ptrs, _stream(stream)), "stq_decode_commit")


def stq_window_flush(pool, slots, stream=None):
    sp, n = _slots(slots, pool)
    _check(_L.stq_window_flush(pool.handle, sp, n, _stream(stream)), "stq_window_flush")


def stq_requant_fixed_scales(pool, slots, stream=None):
    sp, n = _slots(slots, pool)
    _check(_L.stq_requant_fixed_scales(pool.handle, sp, n, _stream(stream)), "stq_requant_fixed_scales")
