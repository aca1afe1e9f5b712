"""qmm_forward launched from a captured HIP graph: every replay (with eager
work and synchronizations between replays) equals the eager call bit for bit,
and meets the oracle bound."""
import numpy as np
import pytest
import torch

import oracle
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


def _replays_equal_eager(run, outs, what):
    """Capture run() (which writes outs), replay it four times with eager work
    and NaN-filled outputs in between, and compare each replay with an eager
    call bit for bit."""
    run()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for rep in range(4):
        for o in outs:
            o.fill_(float("nan"))
        scratch = torch.randn(1 << 16, device=outs[0].device).sum()  # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(scratch)
        for j, (o, e) in enumerate(zip(outs, eager)):
            assert torch.equal(o, e), f"{what}: replay {rep}, output {j} differs from the eager call"
    return eager


@pytest.mark.parametrize("M", [1, 4, 16])
def test_graph_replays_of_the_other_entry_points(M):
    """Split-K (two kernels and a workspace), fused projections, bf16 operands
    and the tiled layout, each captured and replayed like qmm_forward."""
    bits, G, K, N = 4, 32, 1280, 300
    qmm = _gpu.lib()
    o = oracle.get()
    dp = _gpu.DeviceProblem(qmm_inputs.make_problem(seed=60 + M, M=M, K=K, N=N, bits=bits, G=G))
    ref, absum = dp.oracle()
    dev = dp.x.device

    # split-K at S = 3: partials in a workspace, then the in-order sum
    y = torch.empty((M, N), dtype=torch.float32, device=dev)
    ws = torch.empty(qmm.qmm_splitk_workspace_bytes(M, N, 3) // 4, dtype=torch.float32, device=dev)
    (ys,) = _replays_equal_eager(lambda: qmm.qmm_forward_splitk(dp.x, dp.wq, dp.s, dp.b, bits, G, 3,
                                                                 workspace=ws, out=y), [y], "split-K")
    _gpu.assert_parity(ys, ref, absum, f"graph split-K M={M}")

    # two projections of the same x in one launch
    dp2 = _gpu.DeviceProblem(qmm_inputs.make_problem(seed=70 + M, M=M, K=K, N=40, bits=bits, G=G))
    outs = [torch.empty((M, N), dtype=torch.float32, device=dev),
            torch.empty((M, 40), dtype=torch.float32, device=dev)]
    fused = _replays_equal_eager(lambda: qmm.qmm_forward_fused(dp.x, [(dp.wq, dp.s, dp.b), (dp2.wq, dp2.s, dp2.b)],
                                                               bits, G, outs=outs), outs, "fused")
    _gpu.assert_parity(fused[0], ref, absum, f"graph fused M={M}")
    ref2, absum2 = o.forward(dp.p.x, dp2.words, dp2.p.scales, dp2.p.biases, bits, G)
    _gpu.assert_parity(fused[1], ref2, absum2, f"graph fused second projection M={M}")

    # bf16 activations, scales and biases
    db = _gpu.DeviceProblem(qmm_inputs.make_problem(seed=80 + M, M=M, K=K, N=N, bits=bits, G=G, dtype="bf16"))
    yb = torch.empty((M, N), dtype=torch.float32, device=dev)
    (yb_e,) = _replays_equal_eager(lambda: qmm.qmm_forward_bf16(db.x, db.wq, db.s, db.b, bits, G, out=yb),
                                   [yb], "bf16")
    refb, absumb = db.oracle()
    _gpu.assert_parity(yb_e, refb, absumb, f"graph bf16 M={M}")

    # the tiled layout (repacked once, outside the graph)
    tw, tsb = qmm.qmm_repack_tiled(dp.wq, dp.s, dp.b, bits, G)
    yt = torch.empty((M, N), dtype=torch.float32, device=dev)
    (yt_e,) = _replays_equal_eager(lambda: qmm.qmm_forward_tiled(dp.x, tw, tsb, N, bits, G, out=yt), [yt], "tiled")
    _gpu.assert_parity(yt_e, ref, absum, f"graph tiled M={M}")


@pytest.mark.parametrize("M", [4, 16])
def test_graph_replays_of_the_long_k_launch(M):
    """K past the one-pass limit: the fill that clears y and the two K halves
    adding into it, captured together; every replay (y NaN-filled before it)
    equals the eager call bit for bit."""
    bits, G, K, N = 4, 32, 12288, 200
    qmm = _gpu.lib()
    dp = _gpu.DeviceProblem(qmm_inputs.make_problem(seed=90 + M, M=M, K=K, N=N, bits=bits, G=G))
    assert qmm.qmm_kernel_name(M, K, N, bits, G) == "mfma"
    y = torch.empty((M, N), dtype=torch.float32, device=dp.x.device)
    (ye,) = _replays_equal_eager(lambda: qmm.qmm_forward(dp.x, dp.wq, dp.s, dp.b, bits, G, out=y), [y], "long K")
    ref, absum = dp.oracle()
    _gpu.assert_parity(ye, ref, absum, f"graph long K M={M}")
