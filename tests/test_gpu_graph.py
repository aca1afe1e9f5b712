"""qmm_forward launched from a captured HIP graph: every replay (with eager
work and synchronizations between replays) equals the eager call bit for bit,
and meets the oracle bound."""
import numpy as np
import pytest
import torch

import qmm_inputs
from tests import _gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M", [1, 4, 16])
def test_graph_replays_match_eager(M):
    bits, G, K, N = 4, 32, 1280, 300
    dp = _gpu.DeviceProblem(qmm_inputs.make_problem(seed=40 + M, M=M, K=K, N=N, bits=bits, G=G))
    qmm = _gpu.lib()
    eager = qmm.qmm_forward(dp.x, dp.wq, dp.s, dp.b, bits, G)
    torch.cuda.synchronize()
    out = torch.empty_like(eager)
    qmm.qmm_forward(dp.x, dp.wq, dp.s, dp.b, bits, G, out=out)  # warm-up outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        qmm.qmm_forward(dp.x, dp.wq, dp.s, dp.b, bits, G, out=out)
    torch.cuda.synchronize()
    ref, absum = dp.oracle()
    for rep in range(4):
        out.fill_(float("nan"))
        scratch = torch.randn(1 << 16, device=out.device).sum()  # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(scratch)
        assert torch.equal(out, eager), f"replay {rep} differs from the eager call"
        _gpu.assert_parity(out, ref, absum, f"graph replay {rep} M={M}")
