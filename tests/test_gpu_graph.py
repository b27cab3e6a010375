"""Decode steps captured in a HIP graph (as a serving loop or the benchmark's
--graph mode replays them) give, on every replay, exactly what the same
steps give launched one by one: replays separated by eager work and
synchronisations, each checked against an eager twin pool."""
import numpy as np
import pytest

from gpu_util import Pair, say
from workloads import Workload

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("key,B,H", [("C2", 16, 32), ("C5", 8, 4)])
def test_graph_replays_equal_eager(orc, key, B, H):
    import torch
    say("case graph replay", key, B, H)
    wl = Workload(key, B=B, H=H)
    slots = np.arange(B, dtype=np.int32)
    P1, P2 = Pair(orc, wl), Pair(orc, wl)
    S = wl.state(slots)
    P1.store(slots, S)
    P2.store(slots, S)
    sl = P1.slots_t(slots)
    dev = lambda x: torch.as_tensor(x, device="cuda")
    toks = [[dev(x) for x in wl.token(t, n=B)] for t in range(4)]
    o1 = torch.zeros((B, H, wl.dv), dtype=torch.float32, device="cuda")
    o2 = torch.zeros_like(o1)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for tk in toks:
            P2.stq.stq_decode_step(P2.pool, sl, *tk, o2)
    torch.cuda.synchronize()
    assert np.array_equal(P1.image(), P2.image())          # capture runs nothing
    for r in range(3):
        for tk in toks:
            P1.stq.stq_decode_step(P1.pool, sl, *tk, o1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o1, o2), r
        assert np.array_equal(P1.image(), P2.image()), r
        o1.fill_(0.0)                                         # eager work between replays
        torch.cuda.synchronize()
