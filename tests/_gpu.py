"""Helpers shared by the GPU parity tests: move seeded problems to the
device, run the library through its C ABI, compare with the fp64 oracle."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import qmm_inputs


def lib():
    import affine_group_quantized_qmm_amd as qmm  # fails loudly if the library is missing
    return qmm


def dev() -> torch.device:
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    return torch.device("cuda:0")


class DeviceProblem:
    """A seeded problem with its packed words on host and device."""

    def __init__(self, p: qmm_inputs.Problem, pack_on_gpu: bool = True):
        self.p = p
        d = dev()
        qmm = lib()
        o = oracle.get()
        if p.words is not None:
            self.words = p.words
            self.wq = torch.from_numpy(p.words.view(np.int32)).to(d)
        else:
            if pack_on_gpu:
                self.wq = qmm.qmm_pack(torch.from_numpy(p.codes).to(d), p.bits)
                self.words = self.wq.cpu().numpy().view(np.uint32)
            else:
                self.words = o.pack(p.codes, p.bits)
                self.wq = torch.from_numpy(self.words.view(np.int32)).to(d)
        if p.dtype == "bf16":  # uint16 bit patterns -> torch.bfloat16
            def dev_bf16(a):
                return torch.from_numpy(a.view(np.int16)).to(d).view(torch.bfloat16)
            self.x, self.s, self.b = dev_bf16(p.x), dev_bf16(p.scales), dev_bf16(p.biases)
        else:
            self.x = torch.from_numpy(p.x).to(d)
            self.s = torch.from_numpy(p.scales).to(d)
            self.b = torch.from_numpy(p.biases).to(d)

    def oracle(self, rows=None, m_rows=None):
        o = oracle.get()
        x = self.p.x if m_rows is None else self.p.x[m_rows]
        if rows is None:
            return o.forward(x, self.words, self.p.scales, self.p.biases, self.p.bits, self.p.G,
                             dtype=self.p.dtype)
        return o.forward_rows(x, self.words, self.p.scales, self.p.biases, self.p.bits,
                              self.p.G, rows, dtype=self.p.dtype)


def assert_parity(y, ref, absum, label: str) -> float:
    """Element-wise |y - ref| <= 1e-5 * A + 1e-6; returns max err/bound."""
    y = y.detach().cpu().numpy().astype(np.float64) if isinstance(y, torch.Tensor) else y
    assert y.shape == ref.shape, f"{label}: shape {y.shape} != {ref.shape}"
    assert np.isfinite(y).all(), f"{label}: non-finite output"
    err = np.abs(y - ref)
    bound = oracle.parity_bound(absum)
    ratio = err / bound
    worst = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
    assert (err <= bound).all(), (
        f"{label}: {int((err > bound).sum())} of {err.size} outside the bound; worst at {worst}: "
        f"gpu {y[worst]!r} oracle {ref[worst]!r} bound {bound[worst]:.3g}")
    return float(ratio.max())
