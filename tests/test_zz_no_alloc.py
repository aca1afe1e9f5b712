"""qmm_forward_splitk_noalloc (partials in the library's static scratch) against
qmm_forward_splitk with a caller workspace: bitwise equal results, on two
calls in a row, the second with a smaller input, and the scratch limit
rejected on the host."""
import numpy as np
import pytest
import torch

import qmm_inputs
from tests import _gpu

pytestmark = pytest.mark.gpu


def _run_pair(M, K, N, bits, G, split, seed):
    qmm = _gpu.lib()
    dp = _gpu.DeviceProblem(qmm_inputs.make_problem(seed=seed, M=M, K=K, N=N, bits=bits, G=G))
    ws = torch.empty(qmm.qmm_splitk_workspace_bytes(M, N, split) // 4 or 1, dtype=torch.float32,
                     device=dp.x.device)
    want = qmm.qmm_forward_splitk(dp.x, dp.wq, dp.s, dp.b, bits, G, split, workspace=ws)
    got = torch.full((M, N), float("nan"), dtype=torch.float32, device=dp.x.device)
    qmm.qmm_forward_splitk_noalloc(dp.x, dp.wq, dp.s, dp.b, bits, G, split, out=got)
    torch.cuda.synchronize()
    assert torch.equal(got, want), f"M={M} K={K} N={N} S={split}: differs from qmm_forward_splitk"
    ref, absum = dp.oracle()
    _gpu.assert_parity(got, ref, absum, f"noalloc M={M} K={K} N={N} S={split}")


def test_noalloc_two_calls_second_smaller():
    # the long-K down projection shape first (4 slices of 136 groups), then a
    # smaller ragged problem that reuses the same scratch
    _run_pair(16, 17408, 640, 4, 32, 4, seed=1)
    _run_pair(3, 1280, 97, 5, 64, 3, seed=2)


def test_noalloc_single_slice_and_limit():
    qmm = _gpu.lib()
    _run_pair(2, 512, 33, 4, 32, 1, seed=3)
    # partials beyond the scratch: rejected before any launch
    M, K, N, bits, G, split = 16, 8192, 32768, 4, 32, 16
    assert split * M * N * 4 > qmm.QMM_NOALLOC_SCRATCH_BYTES
    dev = _gpu.dev()
    x = torch.zeros((M, K), dtype=torch.float16, device=dev)
    wq = torch.zeros((N, K * bits // 32), dtype=torch.int32, device=dev)
    s = torch.zeros((N, K // G), dtype=torch.float16, device=dev)
    with pytest.raises(qmm.QmmError) as e:
        qmm.qmm_forward_splitk_noalloc(x, wq, s, s, bits, G, split)
    assert e.value.code == qmm.QMM_ERR_SCRATCH
