"""Bitwise admission of multi-row kernels against one-row launches on the
caller's weights (the pages admit a (kind, K, N, rows) only after a bitwise
match and keep the original kernel otherwise)."""
import numpy as np
import pytest
import torch

import qmm_inputs
from tests import _gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,K,N,bits,G", [(2, 1280, 200, 4, 32), (5, 2560, 97, 5, 64), (8, 1024, 64, 8, 128),
                                          (3, 1280, 150, 3, 32), (16, 640, 33, 2, 32)])
def test_rowexact_is_admitted(M, K, N, bits, G):
    qmm = _gpu.lib()
    qmm.qmm_admission_clear()
    dp = _gpu.DeviceProblem(qmm_inputs.make_problem(seed=21, M=M, K=K, N=N, bits=bits, G=G))
    assert qmm.qmm_admission("rowexact", M, K, N, bits, G) == qmm.QMM_ADMISSION_UNKNOWN
    assert qmm.qmm_admit("rowexact", dp.x, dp.wq, dp.s, dp.b, bits, G) is True
    assert qmm.qmm_admission("rowexact", M, K, N, bits, G) == 1
    # the admitted multi-row result is the one-row result, row by row
    y = qmm.qmm_forward_rowexact(dp.x, dp.wq, dp.s, dp.b, bits, G)
    for m in range(M):
        y1 = qmm.qmm_forward_rowexact(dp.x[m:m + 1].contiguous(), dp.wq, dp.s, dp.b, bits, G)
        torch.cuda.synchronize()
        assert torch.equal(y[m:m + 1], y1)
    ref, absum = dp.oracle()
    _gpu.assert_parity(y, ref, absum, f"admitted rowexact M={M}")


def test_forward_admission_follows_the_kernel():
    """qmm_forward's choice is admitted where it is the one-row kernel (M <= 2)
    and rejected where the matrix cores sum in another order (M = 4)."""
    qmm = _gpu.lib()
    qmm.qmm_admission_clear()
    K, N, bits, G = 2560, 300, 4, 32
    p = qmm_inputs.make_problem(seed=22, M=4, K=K, N=N, bits=bits, G=G)
    dp = _gpu.DeviceProblem(p)
    for M, want in ((1, True), (2, True), (4, False)):
        x = dp.x[:M].contiguous()
        got = qmm.qmm_admit("forward", x, dp.wq, dp.s, dp.b, bits, G)
        assert got is want, (M, qmm.qmm_kernel_name(M, K, N, bits, G))
        assert qmm.qmm_admission("forward", M, K, N, bits, G) == int(want)
    qmm.qmm_admission_clear()
    assert qmm.qmm_admission("forward", 4, K, N, bits, G) == qmm.QMM_ADMISSION_UNKNOWN
