"""Tiled (matrix-core) layout: qmm_repack_tiled is bit-exact against the
oracle's repack, and qmm_forward_tiled on the repacked weights meets the
oracle bound of the product on the packed weights."""
import numpy as np
import pytest
import torch

import oracle
import qmm_inputs
from tests import _gpu

pytestmark = pytest.mark.gpu

SHAPES = [(2, 32, 512), (2, 64, 1024), (2, 128, 2048), (4, 32, 512), (4, 64, 1024), (4, 128, 2048),
          (8, 32, 256), (8, 64, 512), (8, 128, 1024), (4, 32, 5120), (8, 32, 4096), (2, 32, 6144)]


@pytest.mark.parametrize("bits,G,K", SHAPES)
def test_repack_bit_exact(bits, G, K):
    qmm = _gpu.lib()
    N = 37  # two full tiles and a ragged third
    dp = _gpu.DeviceProblem(qmm_inputs.make_problem(seed=90 + bits + G, M=1, K=K, N=N, bits=bits, G=G))
    tw, tsb = qmm.qmm_repack_tiled(dp.wq, dp.s, dp.b, bits, G)
    torch.cuda.synchronize()
    want_w, want_sb = oracle.get().repack_tiled(dp.words, dp.p.scales, dp.p.biases, K, bits, G)
    assert np.array_equal(tw.cpu().numpy(), want_w)
    assert np.array_equal(tsb.cpu().numpy().view(np.uint32), want_sb)


@pytest.mark.parametrize("bits,G,K", SHAPES)
@pytest.mark.parametrize("M", [1, 3, 16, 19])
def test_forward_tiled(bits, G, K, M):
    qmm = _gpu.lib()
    N = 150
    dp = _gpu.DeviceProblem(qmm_inputs.make_problem(seed=7 * M + bits + K, M=M, K=K, N=N, bits=bits, G=G))
    tw, tsb = qmm.qmm_repack_tiled(dp.wq, dp.s, dp.b, bits, G)
    y = qmm.qmm_forward_tiled(dp.x, tw, tsb, N, bits, G)
    torch.cuda.synchronize()
    ref, absum = dp.oracle()
    _gpu.assert_parity(y, ref, absum, f"tiled bits={bits} G={G} K={K} M={M}")


@pytest.mark.parametrize("M", [1, 4, 16])
def test_forward_tiled_dense_up(M):
    """The 5120 x 17408 4-bit G=32 projection at full size, checked on a sample of rows."""
    qmm = _gpu.lib()
    K, N = 5120, 17408
    dp = _gpu.DeviceProblem(qmm_inputs.make_problem(seed=3, M=M, K=K, N=N, bits=4, G=32, packed_words=True))
    tw, tsb = qmm.qmm_repack_tiled(dp.wq, dp.s, dp.b, 4, 32)
    y = qmm.qmm_forward_tiled(dp.x, tw, tsb, N, 4, 32)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, N, 211), np.arange(N - 20, N)]))
    ref, absum = dp.oracle(rows=rows)
    _gpu.assert_parity(y[:, rows], ref, absum, f"tiled dense up M={M}")


def test_forward_tiled_rejects_long_k():
    """K = 17408 (4-bit) has a tiled layout but its parts do not fit the kernel."""
    qmm = _gpu.lib()
    dp = _gpu.DeviceProblem(qmm_inputs.make_problem(seed=1, M=2, K=17408, N=16, bits=4, G=32, packed_words=True))
    tw, tsb = qmm.qmm_repack_tiled(dp.wq, dp.s, dp.b, 4, 32)
    with pytest.raises(qmm.QmmError) as e:
        qmm.qmm_forward_tiled(dp.x, tw, tsb, 16, 4, 32)
    assert e.value.code == qmm.QMM_ERR_UNSUPPORTED
