"""The README's usage example runs as written, and its readout is the gated
delta step (A = a S, delta = b (v - A^T k), S' = A + k delta^T, o = S'^T q;
e-cogni STEPQuant analysis, "Contexto") of the states the pool held before
the step, evaluated here in float64 by torch."""
import os
import re

import pytest

from gpu_util import say

pytestmark = pytest.mark.gpu


def test_readme_example_runs():
    import torch
    assert torch.cuda.is_available()
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    blocks = re.findall(r"```python\n(.*?)```", open(os.path.join(root, "README.md")).read(), re.S)
    assert len(blocks) == 1
    say("case README example")
    ns = {}
    exec(compile(blocks[0], "README.md", "exec"), ns)
    Sd, q, k, v, a, b, o, S1 = (ns[x].double().cpu() for x in ("Sd", "q", "k", "v", "a", "b", "o", "S1"))
    A = a[..., None, None] * Sd
    delta = b[..., None] * (v - torch.einsum("chij,chi->chj", A, k))
    Sp = A + k[..., :, None] * delta[..., None, :]
    o_ref = torch.einsum("chij,chi->chj", Sp, q)
    err = float((o - o_ref).abs().max() / o_ref.abs().max())
    say("  README example: readout rel err %.2e" % err)
    assert err < 1e-4
    # the state after the step is requantized to each head's width: relative
    # error of the fetched state about half of these bounds (measured with the
    # oracle on this example: 0.106, 0.025, 0.0062, 0.0002)
    bound = {4: 0.2, 6: 0.05, 8: 0.015, 16: 1e-3}
    for h, n in enumerate(ns["bits"]):
        rel = float((S1[:, h] - Sp[:, h]).norm() / Sp[:, h].norm())
        say("  head %d (%d-bit): refitted state rel err %.2e" % (h, n, rel))
        assert rel < bound[int(n)]
