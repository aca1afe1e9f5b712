"""bfloat16 activations, scales and biases (qmm_forward_bf16) against the fp64
oracle on the same bf16 bit patterns: every bit width and group size, rows
1..17 (the VALU kernel, the matrix-core kernel and several launches), ragged
shapes, rows against one-row calls (bitwise for two-row calls), and the dense
up projection at full size on sampled rows."""
import numpy as np
import pytest
import torch

import qmm_inputs
from qmm_inputs import workloads as W
from tests import _gpu

pytestmark = pytest.mark.gpu

BITS_G = [(b, g) for b in (2, 3, 4, 5, 6, 8) for g in (32, 64, 128)]


@pytest.mark.parametrize("bits,G", BITS_G)
@pytest.mark.parametrize("M", [1, 2, 5, 9, 16])
def test_bf16_small(bits, G, M):
    K, N = 13 * G, 200  # ragged per wave and per workgroup
    dp = _gpu.DeviceProblem(qmm_inputs.make_problem(seed=900 + M * 7 + bits, M=M, K=K, N=N, bits=bits,
                                                    G=G, dtype="bf16"))
    y = _gpu.lib().qmm_forward_bf16(dp.x, dp.wq, dp.s, dp.b, bits, G)
    torch.cuda.synchronize()
    ref, absum = dp.oracle()
    _gpu.assert_parity(y, ref, absum, f"bf16 bits={bits} G={G} M={M}")


@pytest.mark.parametrize("bits,G,K", [(4, 32, 5120), (8, 64, 2048), (5, 64, 2560), (4, 32, 17408),
                                      (2, 128, 4096), (3, 32, 1280)])
def test_bf16_rows_against_one_row_calls(bits, G, K):
    """Every row of a 17-row call and of its one-row calls meets the bound;
    the two rows of a two-row call equal their one-row calls bit for bit."""
    M, N = 17, 150
    dp = _gpu.DeviceProblem(qmm_inputs.make_problem(seed=950 + bits, M=M, K=K, N=N, bits=bits, G=G,
                                                    dtype="bf16"))
    qmm = _gpu.lib()
    y = qmm.qmm_forward_bf16(dp.x, dp.wq, dp.s, dp.b, bits, G)
    y2 = qmm.qmm_forward_bf16(dp.x[:2].contiguous(), dp.wq, dp.s, dp.b, bits, G)
    torch.cuda.synchronize()
    ref, absum = dp.oracle()
    _gpu.assert_parity(y, ref, absum, f"bf16 rows bits={bits} G={G} K={K}")
    for m in range(M):
        y1 = qmm.qmm_forward_bf16(dp.x[m:m + 1].contiguous(), dp.wq, dp.s, dp.b, bits, G)
        torch.cuda.synchronize()
        _gpu.assert_parity(y1, ref[m:m + 1], absum[m:m + 1], f"bf16 row {m} alone")
        if m < 2:
            assert torch.equal(y2[m], y1[0]), f"row {m} of a two-row call differs from its one-row call"


def test_bf16_one_hot_columns():
    """x = e_k for every k: y[k, n] = s[n,k/G] q[n,k] + b[n,k/G] (pins the
    bf16 code widening, its pair order and the scale/bias decode)."""
    for bits, G in ((4, 32), (5, 64), (8, 32), (2, 64)):
        K, N = 2 * G, 40
        p = qmm_inputs.make_problem(seed=5, M=1, K=K, N=N, bits=bits, G=G, dtype="bf16")
        p.x = qmm_inputs.to_bf16_bits(np.eye(K))
        p.M = K
        dp = _gpu.DeviceProblem(p)
        y = _gpu.lib().qmm_forward_bf16(dp.x, dp.wq, dp.s, dp.b, bits, G)
        torch.cuda.synchronize()
        ref, absum = dp.oracle()
        _gpu.assert_parity(y, ref, absum, f"bf16 one-hot bits={bits} G={G}")


@pytest.mark.parametrize("M", [1, 4, 16])
def test_bf16_dense_up_full_size(M):
    s = W.DENSE_UP
    dp = _gpu.DeviceProblem(qmm_inputs.make_problem(seed=0, M=M, K=s.K, N=s.N, bits=s.bits, G=s.G,
                                                    packed_words=True, dtype="bf16"))
    y = _gpu.lib().qmm_forward_bf16(dp.x, dp.wq, dp.s, dp.b, s.bits, s.G)
    torch.cuda.synchronize()
    rng = np.random.default_rng(M)
    rows = np.unique(np.concatenate([rng.choice(s.N, 256, replace=False), [0, 15, 16, s.N - 1]]))
    ref, absum = dp.oracle(rows=rows)
    _gpu.assert_parity(y[:, rows], ref, absum, f"bf16 {s.name} M={M}")


def test_bf16_rejects_fp16_tensors():
    qmm = _gpu.lib()
    dp = _gpu.DeviceProblem(qmm_inputs.make_problem(seed=1, M=1, K=64, N=8, bits=4, G=32))
    with pytest.raises(TypeError):
        qmm.qmm_forward_bf16(dp.x, dp.wq, dp.s, dp.b, 4, 32)


@pytest.mark.parametrize("bits,G,K,M,kernel", [
    (4, 32, 5120, 5, "mfma"),         # register-resident kernel
    (4, 32, 17408, 5, "mfma"),        # several K parts per wave (4 passes)
    (8, 64, 5120, 8, "mfma"),
    (8, 64, 17408, 8, "mfma"),
    (3, 32, 17408, 16, "mfma"),
    (5, 32, 13 * 32, 4, "mfma_lds"),  # rows not whole 16-byte units: LDS-streaming kernel
    (4, 32, 65536, 3, "mfma_lds"),    # more than 8 passes
    (8, 64, 65536, 8, "mfma_lds"),
    (3, 32, 65536, 3, "qmv"),         # neither matrix-core kernel: the VALU kernel
    (6, 64, 5120, 16, "mfma"),
])
def test_bf16_each_kernel_path(bits, G, K, M, kernel):
    """qmm_forward_bf16 takes qmm_forward's kernel; each kernel's bf16 mode
    against the oracle (N = 97: ragged 16-row tiles)."""
    N = 97
    qmm = _gpu.lib()
    assert qmm.qmm_kernel_name(M, K, N, bits, G) == kernel
    dp = _gpu.DeviceProblem(qmm_inputs.make_problem(seed=990 + M + bits, M=M, K=K, N=N, bits=bits, G=G,
                                                    dtype="bf16"))
    y = qmm.qmm_forward_bf16(dp.x, dp.wq, dp.s, dp.b, bits, G)
    torch.cuda.synchronize()
    ref, absum = dp.oracle()
    _gpu.assert_parity(y, ref, absum, f"bf16 {kernel} bits={bits} G={G} K={K} M={M}")
