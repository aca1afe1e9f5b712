"""Fused projections: qmm_forward_fused runs several projections of one x in a
single launch; each output must be bitwise equal to qmm_forward on that
projection alone (same kernel, same per-tile arithmetic) and meet the oracle
bound."""
import numpy as np
import pytest
import torch

import oracle
import qmm_inputs
from tests import _gpu

pytestmark = pytest.mark.gpu


def make_projections(seed, M, K, Ns, bits, G):
    dps = [_gpu.DeviceProblem(qmm_inputs.make_problem(seed=seed + 7 * j, M=M, K=K, N=n, bits=bits, G=G))
           for j, n in enumerate(Ns)]
    return dps[0].x, dps  # every projection reads the first problem's x


@pytest.mark.parametrize("bits,G,K,Ns", [
    (4, 32, 5120, [96, 16, 16]),          # q/k/v-like, whole tiles
    (4, 32, 416, [100, 7, 33, 16]),       # ragged rows, four projections
    (5, 64, 2560, [50, 130]),
    (6, 32, 1280, [17, 1]),
    (8, 128, 2048, [64, 40, 24]),
    (4, 32, 5632, [40, 72]),              # 768-activation parts of the multi-row kernel
    (4, 32, 17408, [33, 20]),             # several K parts per wave
    (4, 32, 65536, [33, 20]),             # more than 8 passes: LDS kernel
    (5, 32, 416, [40, 9]),                # rows not whole 16-byte units: LDS kernel
    (4, 32, 5120, [5120, 1024]),          # alone, the small projection runs as two additive K halves;
    (8, 64, 5120, [2048, 4096]),          # fused, the launch is one slice: the same bits either way
    (4, 32, 5216, [4096, 40]),            # ragged parts: halves only where they match the one-slice parts
])
@pytest.mark.parametrize("M", [1, 2, 3, 8, 16, 19])
def test_fused_equals_separate_calls(bits, G, K, Ns, M):
    qmm = _gpu.lib()
    x, dps = make_projections(300 + M + bits, M, K, Ns, bits, G)
    ys = qmm.qmm_forward_fused(x, [(d.wq, d.s, d.b) for d in dps], bits, G)
    torch.cuda.synchronize()
    for j, (d, y) in enumerate(zip(dps, ys)):
        y1 = qmm.qmm_forward(x, d.wq, d.s, d.b, bits, G)
        torch.cuda.synchronize()
        assert torch.equal(y, y1), f"projection {j} (N={Ns[j]}) differs from its own call"
    if M in (1, 3, 19):
        o = oracle.get()
        for j, (d, y) in enumerate(zip(dps, ys)):
            ref, absum = o.forward(dps[0].p.x, d.words, d.p.scales, d.p.biases, bits, G)
            _gpu.assert_parity(y, ref, absum, f"fused proj {j} bits={bits} G={G} K={K} M={M}")


@pytest.mark.parametrize("M", [1, 8])
def test_fused_qkv_of_a_layer(M):
    """The q/k/v projections of the layer sweep (5120 -> 6144, 1024, 1024) in
    one launch; parity on a sample of columns of each output."""
    qmm = _gpu.lib()
    K, Ns = 5120, [6144, 1024, 1024]
    x, dps = make_projections(4000 + M, M, K, Ns, 4, 32)
    ys = qmm.qmm_forward_fused(x, [(d.wq, d.s, d.b) for d in dps], 4, 32)
    torch.cuda.synchronize()
    o = oracle.get()
    for j, (d, y) in enumerate(zip(dps, ys)):
        assert torch.equal(y, qmm.qmm_forward(x, d.wq, d.s, d.b, 4, 32))
        rows = np.unique(np.concatenate([np.arange(0, Ns[j], 97), [Ns[j] - 1]]))
        ref, absum = o.forward_rows(dps[0].p.x, d.words, d.p.scales, d.p.biases, 4, 32, rows)
        _gpu.assert_parity(y[:, rows], ref, absum, f"qkv proj {j} M={M}")


def test_fused_single_projection_is_forward():
    qmm = _gpu.lib()
    x, dps = make_projections(77, 4, 1024, [200], 4, 32)
    (y,) = qmm.qmm_forward_fused(x, [(dps[0].wq, dps[0].s, dps[0].b)], 4, 32)
    assert torch.equal(y, qmm.qmm_forward(x, dps[0].wq, dps[0].s, dps[0].b, 4, 32))
