"""Parity at the full workload sizes, on sampled output rows that the oracle
computes one by one (same seeded inputs, same entry points and launch
configuration as the benchmark)."""
import numpy as np
import pytest
import torch

import qmm_inputs
from qmm_inputs import workloads as W
from tests import _gpu

pytestmark = pytest.mark.gpu


def sample_rows(N: int, seed: int, count: int = 384) -> np.ndarray:
    rng = np.random.default_rng(seed)
    edges = [0, 1, 15, 16, 63, 64, 65, N // 2, N - 65, N - 64, N - 17, N - 16, N - 2, N - 1]
    rows = np.concatenate([rng.choice(N, size=min(count, N), replace=False), edges])
    return np.unique(np.clip(rows, 0, N - 1))


def run_sampled(dp, y, rows, label, m_rows=None):
    torch.cuda.synchronize()
    ref, absum = dp.oracle(rows=rows, m_rows=m_rows)
    return _gpu.assert_parity(y[:, rows], ref, absum, label)


def test_tiny_full():
    s = W.TINY
    dp = _gpu.DeviceProblem(qmm_inputs.make_problem(seed=0, M=1, K=s.K, N=s.N, bits=s.bits, G=s.G))
    y = _gpu.lib().qmm_forward(dp.x, dp.wq, dp.s, dp.b, s.bits, s.G)
    torch.cuda.synchronize()
    ref, absum = dp.oracle()
    _gpu.assert_parity(y, ref, absum, s.name)


@pytest.fixture(scope="module")
def dense_up():
    s = W.DENSE_UP
    return _gpu.DeviceProblem(qmm_inputs.make_problem(
        seed=0, M=max(W.DENSE_UP_M), K=s.K, N=s.N, bits=s.bits, G=s.G, packed_words=True))


@pytest.mark.parametrize("M", W.DENSE_UP_M)
def test_dense_up(dense_up, M):
    s = W.DENSE_UP
    x = dense_up.x[:M].contiguous()
    y = _gpu.lib().qmm_forward(x, dense_up.wq, dense_up.s, dense_up.b, s.bits, s.G)
    run_sampled(dense_up, y, sample_rows(s.N, M), f"{s.name} M={M}", m_rows=slice(0, M))


@pytest.mark.parametrize("shape", W.MIXED, ids=lambda s: s.name)
def test_mixed_bits(shape):
    s = shape
    dp = _gpu.DeviceProblem(qmm_inputs.make_problem(
        seed=s.bits, M=max(W.MIXED_M), K=s.K, N=s.N, bits=s.bits, G=s.G))
    for M in W.MIXED_M:
        y = _gpu.lib().qmm_forward(dp.x[:M].contiguous(), dp.wq, dp.s, dp.b, s.bits, s.G)
        run_sampled(dp, y, sample_rows(s.N, M), f"{s.name} M={M}", m_rows=slice(0, M))


@pytest.mark.parametrize("S", W.LONG_K_SPLITS)
def test_long_k_splitk(S):
    s = W.LONG_K
    dp = _gpu.DeviceProblem(qmm_inputs.make_problem(
        seed=0, M=W.LONG_K_M, K=s.K, N=s.N, bits=s.bits, G=s.G, packed_words=True))
    y = _gpu.lib().qmm_forward_splitk(dp.x, dp.wq, dp.s, dp.b, s.bits, s.G, S)
    run_sampled(dp, y, sample_rows(s.N, S), f"{s.name} S={S}")


@pytest.mark.parametrize("M", W.SWEEP_M)
def test_one_sweep_layer(M):
    for layer, j, s, seed in W.sweep_shapes(layers=1):
        dp = _gpu.DeviceProblem(qmm_inputs.make_problem(
            seed=seed, M=M, K=s.K, N=s.N, bits=s.bits, G=s.G, packed_words=True))
        y = _gpu.lib().qmm_forward(dp.x, dp.wq, dp.s, dp.b, s.bits, s.G)
        run_sampled(dp, y, sample_rows(s.N, seed, count=128), f"{s.name} M={M}")
