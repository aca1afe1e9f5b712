"""Row-exact mode: every row of an M-row qmm_forward_rowexact call is bitwise
equal to the one-row qmm_forward on that row (the row-batched kernel keeps the
one-row statement order), and meets the oracle bound."""
import pytest
import torch

import qmm_inputs
from tests import _gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("bits,G,K", [(4, 32, 5120), (4, 32, 416), (5, 64, 2560), (6, 32, 1280),
                                      (8, 128, 2048), (4, 32, 17408), (4, 64, 8192),
                                      # groups of 40+ bytes: the one-row launch loads them coalesced
                                      # through LDS (several K chunks; 9280 x 5 bits leaves rows not
                                      # 16-byte aligned, which takes the per-lane loads)
                                      (8, 64, 17408), (6, 128, 8448), (5, 64, 9280)])
@pytest.mark.parametrize("M", [2, 3, 5, 8, 11])
def test_rows_bitwise_equal_one_row_calls(bits, G, K, M):
    N = 150
    dp = _gpu.DeviceProblem(qmm_inputs.make_problem(seed=60 + M + bits, M=M, K=K, N=N, bits=bits, G=G))
    qmm = _gpu.lib()
    y = qmm.qmm_forward_rowexact(dp.x, dp.wq, dp.s, dp.b, bits, G)
    torch.cuda.synchronize()
    for m in range(M):
        y1 = qmm.qmm_forward(dp.x[m:m + 1].contiguous(), dp.wq, dp.s, dp.b, bits, G)
        torch.cuda.synchronize()
        assert torch.equal(y[m], y1[0]), f"row {m} of {M} differs from its one-row call"
    ref, absum = dp.oracle()
    _gpu.assert_parity(y, ref, absum, f"rowexact bits={bits} G={G} K={K} M={M}")


def test_rowexact_rejects_like_forward():
    """Argument errors come back as the same codes as qmm_forward, before any launch."""
    qmm = _gpu.lib()
    dp = _gpu.DeviceProblem(qmm_inputs.make_problem(seed=1, M=2, K=64, N=8, bits=4, G=32))
    y = torch.empty((2, 8), dtype=torch.float32, device=dp.x.device)
    ptrs = (dp.x.data_ptr(), dp.wq.data_ptr(), dp.s.data_ptr(), dp.b.data_ptr(), y.data_ptr())
    stream = torch.cuda.current_stream().cuda_stream
    for bits, G, code in ((7, 32, -3), (4, 48, -4)):
        assert qmm._lib.qmm_forward_rowexact(*ptrs, 2, 64, 8, bits, G, stream) == code
        assert qmm._lib.qmm_forward(*ptrs, 2, 64, 8, bits, G, stream) == code
