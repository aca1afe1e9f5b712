"""qmm_forward (and each kernel forced by name) against the fp64 oracle on
seeded inputs: every bit width and group size, activation rows 1..33, shapes
spanning several tiles with ragged tails, single-group and chunk-boundary K."""
import numpy as np
import pytest
import torch

import qmm_inputs
from tests import _gpu

pytestmark = pytest.mark.gpu

BITS_G = [(b, g) for b in (2, 3, 4, 5, 6, 8) for g in (32, 64, 128)]


@pytest.mark.parametrize("bits,G", BITS_G)
@pytest.mark.parametrize("M", [1, 2, 3, 8, 16])
def test_forward_small(bits, G, M):
    # N = 200: three 64-row workgroups plus a ragged tail; K = 13 groups (ragged per wave)
    K, N = 13 * G, 200
    dp = _gpu.DeviceProblem(qmm_inputs.make_problem(seed=M * 7 + bits, M=M, K=K, N=N, bits=bits, G=G))
    qmm = _gpu.lib()
    y = qmm.qmm_forward(dp.x, dp.wq, dp.s, dp.b, bits, G)
    torch.cuda.synchronize()
    ref, absum = dp.oracle()
    _gpu.assert_parity(y, ref, absum, f"forward bits={bits} G={G} M={M}")


KERNELS = ["qmv", "mfma", "mfma_lds"]


def run_kernel(kernel, dp, bits, G):
    """Forced-kernel call; "mfma" on a shape it cannot run (and "mfma_lds" on
    3-bit codes at G = 32) must say so, and then qmm_forward must not pick it."""
    qmm = _gpu.lib()
    try:
        return qmm.qmm_forward_kernel(kernel, dp.x, dp.wq, dp.s, dp.b, bits, G)
    except qmm.QmmError as e:
        assert e.code == qmm.QMM_ERR_UNSUPPORTED, str(e)
        assert kernel == "mfma" or (kernel == "mfma_lds" and (bits, G) == (3, 32)), str(e)
        M, K, N = dp.p.M, dp.p.K, dp.p.N
        assert qmm.qmm_kernel_name(max(M, 3), K, N, bits, G) != kernel
        return None


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("M", [1, 4, 16])
@pytest.mark.parametrize("bits,G,K", [(4, 32, 1280), (5, 64, 2560), (6, 32, 1280), (8, 128, 2048),
                                      (8, 64, 4096), (2, 32, 1280), (2, 128, 4096), (3, 32, 1280),
                                      (3, 64, 2560)])
def test_each_kernel(kernel, M, bits, G, K):
    N = 97
    dp = _gpu.DeviceProblem(qmm_inputs.make_problem(seed=11, M=M, K=K, N=N, bits=bits, G=G))
    y = run_kernel(kernel, dp, bits, G)
    if (kernel, bits, G) == ("mfma_lds", 3, 32):
        assert y is None
        return
    assert y is not None, f"{kernel} should support bits={bits} G={G} K={K}"
    torch.cuda.synchronize()
    ref, absum = dp.oracle()
    _gpu.assert_parity(y, ref, absum, f"{kernel} bits={bits} G={G} M={M}")


@pytest.mark.parametrize("M", [17, 33])
def test_more_than_16_rows(M):
    bits, G, K, N = 4, 32, 1024, 130
    dp = _gpu.DeviceProblem(qmm_inputs.make_problem(seed=M, M=M, K=K, N=N, bits=bits, G=G))
    y = _gpu.lib().qmm_forward(dp.x, dp.wq, dp.s, dp.b, bits, G)
    torch.cuda.synchronize()
    ref, absum = dp.oracle()
    _gpu.assert_parity(y, ref, absum, f"M={M}")


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("K,N", [(32, 1), (32, 64), (64, 5), (6144, 19), (6176, 23), (8192, 33),
                                 (8192 + 32, 17), (17408, 9)])
def test_edge_shapes(kernel, K, N):
    """Single group, single row, one chunk exactly, one group past a chunk, the
    longest K the register-resident kernel takes and one group more, long K."""
    bits, G = 4, 32
    for M in (1, 5):
        dp = _gpu.DeviceProblem(qmm_inputs.make_problem(seed=K + N + M, M=M, K=K, N=N, bits=bits, G=G))
        y = run_kernel(kernel, dp, bits, G)
        if y is None:
            continue
        torch.cuda.synchronize()
        ref, absum = dp.oracle()
        _gpu.assert_parity(y, ref, absum, f"{kernel} K={K} N={N} M={M}")


@pytest.mark.parametrize("bits,G", [(4, 32), (5, 32), (6, 64), (8, 32)])
def test_one_hot_columns(bits, G):
    """x = e_k for every k: y[k, n] = s[n,k/G] q[n,k] + b[n,k/G] (pins column/bit order)."""
    K, N = 4 * G, 70
    p = qmm_inputs.make_problem(seed=5, M=1, K=K, N=N, bits=bits, G=G)
    p.x = np.eye(K, dtype=np.float16)
    p.M = K
    dp = _gpu.DeviceProblem(p)
    qmm = _gpu.lib()
    for kernel in KERNELS:
        y = qmm.qmm_forward_kernel(kernel, dp.x, dp.wq, dp.s, dp.b, bits, G)
        torch.cuda.synchronize()
        ref, absum = dp.oracle()
        _gpu.assert_parity(y, ref, absum, f"one-hot {kernel} bits={bits}")


def test_rows_agree_with_single_row_calls():
    """Each row of an M-row call meets the bound on its own; report bitwise equality to M=1."""
    bits, G, K, N, M = 4, 32, 2048, 300, 8
    dp = _gpu.DeviceProblem(qmm_inputs.make_problem(seed=3, M=M, K=K, N=N, bits=bits, G=G))
    qmm = _gpu.lib()
    y = qmm.qmm_forward(dp.x, dp.wq, dp.s, dp.b, bits, G)
    ref, absum = dp.oracle()
    same = 0
    for m in range(M):
        y1 = qmm.qmm_forward(dp.x[m:m + 1].contiguous(), dp.wq, dp.s, dp.b, bits, G)
        torch.cuda.synchronize()
        _gpu.assert_parity(y1, ref[m:m + 1], absum[m:m + 1], f"row {m} alone")
        same += int(torch.equal(y1[0], y[m]))
    _gpu.assert_parity(y, ref, absum, "all rows")
    print(f"rows bitwise equal to their 1-row call: {same} of {M}")


def test_deterministic_rerun():
    bits, G, K, N, M = 5, 64, 5120, 256, 4
    dp = _gpu.DeviceProblem(qmm_inputs.make_problem(seed=9, M=M, K=K, N=N, bits=bits, G=G))
    qmm = _gpu.lib()
    a = qmm.qmm_forward(dp.x, dp.wq, dp.s, dp.b, bits, G)
    b = qmm.qmm_forward(dp.x, dp.wq, dp.s, dp.b, bits, G)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("bits,G,K,N,M", [(4, 32, 17408, 336, 5), (8, 64, 17408, 336, 5), (3, 32, 17408, 336, 5),
                                          (4, 32, 6176, 1, 3), (4, 32, 6176, 17, 16), (5, 64, 6272, 40, 8),
                                          (2, 32, 12288, 50, 4)])
def test_long_k_two_halves(bits, G, K, N, M):
    """K too long for one pass of the matrix-core kernel (from just past the
    one-pass limit on): the two K halves add into y, which the call clears
    first (y starts as NaN here). Two addends per output, so reruns are
    bitwise identical; parity with the oracle; N down to one column."""
    dp = _gpu.DeviceProblem(qmm_inputs.make_problem(seed=23, M=M, K=K, N=N, bits=bits, G=G))
    qmm = _gpu.lib()
    assert qmm.qmm_kernel_name(M, K, N, bits, G) == "mfma"
    outs = []
    for _ in range(4):
        y = torch.full((M, N), float("nan"), dtype=torch.float32, device=dp.x.device)
        outs.append(qmm.qmm_forward(dp.x, dp.wq, dp.s, dp.b, bits, G, out=y))
    torch.cuda.synchronize()
    ref, absum = dp.oracle()
    _gpu.assert_parity(outs[0], ref, absum, f"long K bits={bits} G={G}")
    for y in outs[1:]:
        assert torch.equal(y, outs[0])


def test_rejects_misaligned_tensor():
    qmm = _gpu.lib()
    bits, G, K, N = 4, 32, 256, 64
    dp = _gpu.DeviceProblem(qmm_inputs.make_problem(seed=1, M=2, K=K + G, N=N, bits=bits, G=G))
    x_off = dp.x.view(-1)[1:1 + 2 * K].view(2, K)  # 2-byte offset
    with pytest.raises(qmm.QmmError) as e:
        qmm.qmm_forward(x_off, dp.wq[:, :K * bits // 32].contiguous(), dp.s[:, :K // G].contiguous(),
                        dp.b[:, :K // G].contiguous(), bits, G)
    assert e.value.code == -7
