"""qmm_pack on the GPU is bit-exact against the oracle's pack."""
import numpy as np
import pytest
import torch

import oracle
from tests import _gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 8])
@pytest.mark.parametrize("N,K", [(1, 32), (3, 64), (17, 96), (64, 512), (129, 1056), (5, 5120)])
def test_pack_bit_exact(bits, N, K):
    qmm = _gpu.lib()
    rng = np.random.default_rng(1000 * bits + N)
    codes = rng.integers(0, 1 << bits, size=(N, K), dtype=np.uint8)
    packed = qmm.qmm_pack(torch.from_numpy(codes).to(_gpu.dev()), bits)
    torch.cuda.synchronize()
    got = packed.cpu().numpy().view(np.uint32)
    assert np.array_equal(got, oracle.get().pack(codes, bits))


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 8])
def test_pack_ignores_high_bits(bits):
    """Bits above `bits` in an input byte are not stored."""
    qmm = _gpu.lib()
    rng = np.random.default_rng(bits)
    codes = rng.integers(0, 256, size=(9, 128), dtype=np.uint8)
    packed = qmm.qmm_pack(torch.from_numpy(codes).to(_gpu.dev()), bits)
    torch.cuda.synchronize()
    want = oracle.get().pack(codes & np.uint8((1 << bits) - 1), bits)
    assert np.array_equal(packed.cpu().numpy().view(np.uint32), want)
