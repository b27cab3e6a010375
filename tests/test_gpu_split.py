"""The decode step split in two (stq_decode_readout + stq_decode_commit),
through the C ABI: the pair gives exactly the fused step's readout and bytes
(bit for bit), on one stream and with the commit on a second stream ordered by
events over several tokens; the readout matches the oracle's step to the
decode bar and leaves the pool untouched; unsupported pools are refused."""
import numpy as np
import pytest

from gpu_util import Pair, readout_ok, say
from workloads import Workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available()
    return torch


def _pools(orc, key, B, H):
    wl = Workload(key, B=B, H=H)
    slots = np.random.default_rng(B).permutation(B + 2)[:B].astype(np.int32)
    P1, P2 = Pair(orc, wl, n_slots=B + 2), Pair(orc, wl, n_slots=B + 2)
    S = wl.state(slots)
    P1.store(slots, S)
    P2.store(slots, S)
    assert np.array_equal(P1.image(), P2.image())
    return wl, slots, P1, P2


@pytest.mark.parametrize("key,B,H", [("C1", 4, 2), ("C2", 24, 32), ("C3", 16, 32)])
def test_split_equals_fused_one_stream(torch_cuda, orc, key, B, H):
    torch = torch_cuda
    say("case split one stream", key, B, H)
    wl, slots, P1, P2 = _pools(orc, key, B, H)
    dev = lambda x: torch.as_tensor(x, device="cuda")
    sl = P1.slots_t(slots)
    for t in range(3):
        q, k, v, a, b = [dev(x) for x in wl.token(t, n=B)]
        pre = P2.image()
        o1 = torch.empty((B, H, wl.dv), dtype=torch.float32, device="cuda")
        o2 = torch.empty_like(o1)
        P1.stq.stq_decode_step(P1.pool, sl, q, k, v, a, b, o1)
        P2.stq.stq_decode_readout(P2.pool, sl, q, k, v, a, b, o2)
        assert np.array_equal(P2.image(), pre)                   # the readout writes no tile
        P2.stq.stq_decode_commit(P2.pool, sl, q, k, v, a, b)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2)
        assert np.array_equal(P1.image(), P2.image())
        ref = orc.OraclePool(P2.n_slots, H, wl.dk, wl.dv, wl.bits, wl.row_weight, image=pre)
        o_ref = ref.step(slots, *[x.cpu().numpy() for x in (q, k, v, a, b)])
        assert readout_ok(o2.cpu().numpy(), o_ref) <= 1.0


def test_split_two_streams(torch_cuda, orc):
    torch = torch_cuda
    say("case split two streams")
    B, H = 32, 32
    wl, slots, P1, P2 = _pools(orc, "C2", B, H)
    dev = lambda x: torch.as_tensor(x, device="cuda")
    sl = P1.slots_t(slots)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    toks = [[dev(x) for x in wl.token(t, n=B)] for t in range(6)]
    torch.cuda.synchronize()
    o1 = [torch.empty((B, H, wl.dv), dtype=torch.float32, device="cuda") for _ in toks]
    o2 = [torch.empty_like(x) for x in o1]
    for t, tk in enumerate(toks):
        P1.stq.stq_decode_step(P1.pool, sl, *tk, o1[t])
    done = None
    for t, tk in enumerate(toks):
        if done is not None:
            sa.wait_event(done)
        P2.stq.stq_decode_readout(P2.pool, sl, *tk, o2[t], stream=sa)
        read = torch.cuda.Event()
        read.record(sa)
        sb.wait_event(read)
        P2.stq.stq_decode_commit(P2.pool, sl, *tk, stream=sb)
        done = torch.cuda.Event()
        done.record(sb)
    torch.cuda.synchronize()
    for t in range(len(toks)):
        assert torch.equal(o1[t], o2[t]), t
    assert np.array_equal(P1.image(), P2.image())


def test_split_unsupported(torch_cuda, orc):
    torch = torch_cuda
    import quantized_linear_attention_amd as stq
    say("case split unsupported")
    f = lambda *s: torch.zeros(s, dtype=torch.float32, device="cuda")
    for key in ("C4", "C5"):
        wl = Workload(key, B=1, H=2)
        P = Pair(orc, wl, n_slots=1)
        dk, dv = wl.dk, wl.dv
        q, k, v, o = f(2 * dk), f(2 * dk), f(2 * dv), f(2 * dv)
        a, b = f(2 * (dk if wl.cfg.gate else 1)), f(2)
        with pytest.raises(stq.StqError) as e:
            stq.stq_decode_readout(P.pool, P.slots_t([0]), q, k, v, a, b, o)
        assert e.value.status == -5
        with pytest.raises(stq.StqError) as e:
            stq.stq_decode_commit(P.pool, P.slots_t([0]), q, k, v, a, b)
        assert e.value.status == -5
