"""CPU-side checks of the C ABI: the library loads, exports every entry
point declared in include/stq.h, sizes pools like the (independent) oracle,
and rejects bad arguments on the host before touching the GPU."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    txt = open(os.path.join(ROOT, "include", "stq.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(stq_[a-z_]+)\s*\(", txt)))


@pytest.fixture(scope="module")
def stq():
    import quantized_linear_attention_amd as q
    return q


def test_exports_every_declared_symbol(stq):
    names = _declared()
    assert "stq_decode_step" in names and "stq_window_flush" in names and "stq_pool_create" in names
    lib = ctypes.CDLL(stq.library_path())
    for n in names:
        assert hasattr(lib, n), n


@pytest.mark.parametrize("key,B", [("C1", 4), ("C2", 64), ("C3", 512), ("C4", 256), ("C5", 512)])
def test_pool_bytes_agree_with_oracle(stq, orc, key, B):
    from workloads import Workload
    wl = Workload(key, B=B)
    bits = np.asarray(wl.bits).reshape(-1)
    d = stq.make_desc(B, wl.H, wl.dk, wl.dv, bits, wl.row_weight, wl.cfg.gate, wl.cfg.unit,
                      wl.cfg.window)
    P = orc.OraclePool(B, wl.H, wl.dk, wl.dv, bits, wl.row_weight, wl.cfg.gate, wl.cfg.unit,
                       wl.cfg.window)
    assert stq.stq_pool_bytes(d) == P.nbytes


def test_c3_pool_size(stq):
    from workloads import Workload
    wl = Workload("C3")
    d = stq.make_desc(512, 32, 128, 128, wl.bits, wl.row_weight)
    n = stq.stq_pool_bytes(d)
    assert n - 512 * 417280 < 64 * 1024                 # header is small
    assert 512 * 417280 == 213647360                    # 213.6 MB of packed state


def test_invalid_descriptors(stq):
    ok = dict(n_slots=2, n_heads=2, d_k=128, d_v=128, unit_bits=[6, 6], row_weight=np.ones(256))
    assert stq.stq_pool_bytes(stq.make_desc(**ok)) > 0
    bad = [dict(ok, n_slots=0), dict(ok, d_k=96), dict(ok, d_v=32), dict(ok, unit_bits=[6, 5]),
           dict(ok, row_weight=np.r_[np.ones(255), 0.0]), dict(ok, row_weight=np.r_[np.ones(255), np.nan]),
           dict(ok, window=64), dict(ok, gate_kind=3),
           dict(ok, n_comp=2), dict(ok, window=8, n_comp=9), dict(ok, window=30, n_comp=3),
           dict(ok, window=8, n_comp=-1)]
    for b in bad:
        assert stq.stq_pool_bytes(stq.make_desc(**b)) == 0


def test_compensator_cache_layout(stq, orc):
    """Window caches grow by n_comp binary32 rows of d_v; the header keeps
    W | n_comp << 16; sizes agree with the oracle's layout."""
    base = dict(n_slots=3, n_heads=2, d_k=128, d_v=64, unit_bits=[6, 16], row_weight=np.ones(256), window=8)
    n0 = stq.stq_pool_bytes(stq.make_desc(**base))
    n4 = stq.stq_pool_bytes(stq.make_desc(**dict(base, n_comp=4)))
    assert n4 - n0 == 3 * 2 * 4 * 4 * 64
    ref = orc.OraclePool(3, 2, 128, 64, np.array([6, 16]), np.ones((2, 128)), window=8, n_comp=4)
    assert ref.nbytes == n4
    assert int(ref.img[28:32].view(np.uint32)[0]) == 8 | (4 << 16)


def test_create_rejects_on_host(stq):
    lib = ctypes.CDLL(stq.library_path())
    lib.stq_pool_create.restype = ctypes.c_int32
    d = stq.make_desc(2, 2, 128, 128, [6, 6], np.ones(256))
    out = ctypes.c_void_p()
    need = stq.stq_pool_bytes(d)
    # misaligned device pointer / too small: layout errors, nothing enqueued
    r = lib.stq_pool_create(ctypes.byref(d), ctypes.c_void_p(0x1001), ctypes.c_size_t(need), None, ctypes.byref(out))
    assert r == -2 and not out.value
    r = lib.stq_pool_create(ctypes.byref(d), ctypes.c_void_p(0x10000), ctypes.c_size_t(need - 1), None, ctypes.byref(out))
    assert r == -2
    bad = stq.make_desc(2, 2, 128, 128, [6, 7], np.ones(256))
    r = lib.stq_pool_create(ctypes.byref(bad), ctypes.c_void_p(0x10000), ctypes.c_size_t(need), None, ctypes.byref(out))
    assert r == -1
    assert "LAYOUT" in stq.stq_status_str(-2)


def test_prefill_rejects_on_host(stq):
    """A null pool handle is refused before anything is enqueued."""
    lib = ctypes.CDLL(stq.library_path())
    lib.stq_prefill.restype = ctypes.c_int32
    P = ctypes.c_void_p
    lib.stq_prefill.argtypes = [P, P, ctypes.c_int32] + [P] * 7 + [P]
    r = lib.stq_prefill(None, P(0x10000), 1, P(0x10000), P(0x10000), P(0x10000), P(0x10000),
                        P(0x10000), P(0x10000), P(0x10000), None)
    assert r == -1


def test_new_entry_points_reject_on_host(stq):
    """Bad sizes, kinds or handles are refused on the host before anything is enqueued."""
    lib = ctypes.CDLL(stq.library_path())
    P, I = ctypes.c_void_p, ctypes.c_int32
    lib.stq_prefill_states.restype = I
    lib.stq_prefill_states.argtypes = [I, I, I, I, I] + [P] * 8 + [P]
    d = P(0x10000)
    args = [d] * 8
    for n, H, dk, dv, gate in [(-1, 2, 128, 128, 0), (1, 0, 128, 128, 0), (1, 4097, 128, 128, 0),
                               (1, 2, 96, 128, 0), (1, 2, 128, 32, 0), (1, 2, 128, 128, 2)]:
        assert lib.stq_prefill_states(n, H, dk, dv, gate, *args, None) == -1
    assert lib.stq_prefill_states(1, 2, 128, 128, 0, None, *args[1:], None) == -1
    assert lib.stq_prefill_states(0, 2, 128, 128, 0, *args, None) == 0          # nothing to do
    for name, npt in (("stq_decode_readout", 7), ("stq_decode_commit", 6)):
        f = getattr(lib, name)
        f.restype = I
        f.argtypes = [P, P, I] + [P] * npt + [P]
        assert f(None, d, 1, *([d] * npt), None) == -1


class _FakeCuda:
    """Stands in for a CUDA tensor on a machine without a GPU: the binding's
    size and device checks run before any pointer reaches the library."""
    def __init__(self, numel, dtype, device="cuda:0"):
        import torch
        self._n, self.dtype, self.device = numel, dtype, torch.device(device)
        self.is_cuda = True

    def is_contiguous(self):
        return True

    def numel(self):
        return self._n

    def data_ptr(self):
        return 0x10000

    def dim(self):
        return 1


def _fake_pool(stq, gate=0, window=0):
    import torch
    from quantized_linear_attention_amd import _lib
    d = stq.make_desc(4, 2, 128, 64, [6, 8], np.ones(256), gate, 0, window)
    return _lib._Pool(None, d, _FakeCuda(1 << 20, torch.uint8))


@pytest.mark.parametrize("gate", [0, 1])
def test_binding_rejects_short_or_misplaced_tensors(stq, gate):
    """Every per-token tensor is checked against the pool's sizes (q, k: n H d_k;
    v, o: n H d_v; a: n H or n H d_k by gate kind; b: n H; S: n H d_k d_v) and
    the pool buffer's device before the library is called."""
    import torch
    f = torch.float32
    pool = _fake_pool(stq, gate)
    n, H, dk, dv = 3, 2, 128, 64
    good = dict(q=n * H * dk, k=n * H * dk, v=n * H * dv, a=n * H * (dk if gate else 1), b=n * H, o=n * H * dv)
    slots = _FakeCuda(n, torch.int32)
    for name in good:
        for wrong in (good[name] - 1, good[name] + 1):
            args = {k: _FakeCuda(v, f) for k, v in good.items()}
            args[name] = _FakeCuda(wrong, f)
            with pytest.raises(stq.StqError, match=name):
                stq.stq_decode_step(pool, slots, **args)
            if name != "o":
                with pytest.raises(stq.StqError, match=name):
                    stq.stq_decode_commit(pool, slots, *[args[k] for k in "qkvab"])
            with pytest.raises(stq.StqError, match=name):
                stq.stq_decode_readout(pool, slots, **args)
    # a per-head gate where the pool wants per-channel gates, and the reverse
    other = n * H * (1 if gate else dk)
    args = {k: _FakeCuda(v, f) for k, v in good.items()}
    args["a"] = _FakeCuda(other, f)
    with pytest.raises(stq.StqError, match="a has"):
        stq.stq_decode_step(pool, slots, **args)
    # another device than the pool buffer's
    args = {k: _FakeCuda(v, f) for k, v in good.items()}
    args["v"] = _FakeCuda(good["v"], f, "cuda:1")
    with pytest.raises(stq.StqError, match="cuda:1"):
        stq.stq_decode_step(pool, slots, **args)
    with pytest.raises(stq.StqError, match="cuda:1"):
        stq.stq_decode_step(pool, _FakeCuda(n, torch.int32, "cuda:1"), **{k: _FakeCuda(v, f) for k, v in good.items()})
    # store / fetch: the whole state
    for fn in (stq.stq_pool_store, stq.stq_pool_fetch):
        with pytest.raises(stq.StqError, match="S has"):
            fn(pool, slots, _FakeCuda(n * H * dk * dv - 1, f))


def test_binding_rejects_bad_prompt_offsets(stq):
    """Prefill: seq_start needs n + 1 entries; q must be whole tokens."""
    import torch
    f = torch.float32
    pool = _fake_pool(stq)
    slots = _FakeCuda(3, torch.int32)
    tok = 10
    sizes = dict(q=tok * 2 * 128, k=tok * 2 * 128, v=tok * 2 * 64, a=tok * 2, b=tok * 2, o=tok * 2 * 64)
    args = {k: _FakeCuda(v, f) for k, v in sizes.items()}
    with pytest.raises(stq.StqError, match="seq_start"):
        stq.stq_prefill(pool, slots, _FakeCuda(3, torch.int32), **args)
    args["q"] = _FakeCuda(sizes["q"] + 5, f)
    with pytest.raises(stq.StqError, match="q must be"):
        stq.stq_prefill(pool, slots, _FakeCuda(4, torch.int32), **args)
