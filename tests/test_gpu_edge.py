"""Degenerate inputs of the method on every entry point, against the fp64 oracle.

Rows of the weight matrix where the factored form s*P + b*XS has nothing to
add or cancels exactly, and activation rows at the extremes of fp16:

* zero-weight rows: every code 0 and every bias 0, scales non-zero (w = 0);
* rows with every scale 0 (w = b: only the bias term b*XS remains);
* saturated rows: every code 2^bits - 1 with b = -s*(2^bits - 1) exactly
  (s a power of two), so that w = s*q + b = 0 although s*P and b*XS are
  both large;
* activation rows of zeros, and rows with |x| near the fp16 maximum.

Where w = 0 the oracle's absolute sum A = sum_k |w x| is 0 and the bound is
the absolute 1e-6 alone; the kernels widen codes exactly (no offset carried
through the dot product), so zero-weight rows come out as exactly 0.
Saturated rows cancel, in every group, two fp32 terms of size
s*(2^bits - 1)*|XS| each, so the error of any fp32 evaluation of the
factored form on them is a few rounding units of those terms, summed over
the K/G groups, against an absolute bound of 1e-6. They are tested with the
bias in the middle of the workloads' bias range (s*(2^bits - 1) = 1/16 up
to a power of two) and with activations of the workloads' scale (N(0, 1)
and zero rows). Activations near the fp16 maximum are tested against the
other rows (random, zero-weight, zero-scale).
"""
import numpy as np
import pytest
import torch

import qmm_inputs
from tests import _gpu

pytestmark = pytest.mark.gpu

# (bits, G, power-of-two scale of the saturated rows: s * (2^bits - 1) about 1/16,
#  so that b = -s * (2^bits - 1) lies in the middle of the bias range U(-0.1, 0.1))
CASES = [(4, 32, 2.0 ** -8), (2, 32, 2.0 ** -6), (5, 64, 2.0 ** -9), (8, 64, 2.0 ** -12)]
K_GROUPS = 40          # K = 40 groups: whole 16-byte rows for every width, several K parts
N = 97                 # ragged: 6 tiles of 16 rows plus one row
ZERO_ROWS = range(0, 6)
SZERO_ROWS = range(6, 12)
SAT_ROWS = range(40, 46)


def _round(a, dtype):
    return a.astype(np.float16) if dtype == "f16" else qmm_inputs.to_bf16_bits(a)


X_KINDS = {"random": ("random",), "zero": ("zero",), "large": ("large",),
           "mixed": ("random", "zero"), "mixed_large": ("random", "large", "zero")}


def edge_problem(bits, G, M, x_case, seed, dtype="f16"):
    """A seeded problem whose weight rows include the degenerate rows above and
    whose activation rows follow `x_case` (a key of X_KINDS: activation row m
    takes kind m % len(kinds)). Saturated rows are present unless an
    activation row is large."""
    K = K_GROUPS * G
    p = qmm_inputs.make_problem(seed=seed, M=M, K=K, N=N, bits=bits, G=G, dtype=dtype)
    rng = np.random.default_rng(seed + 1)
    Kg = K // G
    codes = p.codes.copy()
    s64 = rng.uniform(*qmm_inputs.SCALE_RANGE, size=(N, Kg))
    b64 = rng.uniform(*qmm_inputs.BIAS_RANGE, size=(N, Kg))
    for r in ZERO_ROWS:
        codes[r] = 0
        b64[r] = 0.0
    for r in SZERO_ROWS:
        s64[r] = 0.0
    kinds = X_KINDS[x_case]
    row_kinds = [kinds[m % len(kinds)] for m in range(M)]
    if "large" not in row_kinds:
        _, _, s_sat = next(c for c in CASES if c[:2] == (bits, G))
        qmax = (1 << bits) - 1
        for r in SAT_ROWS:
            codes[r] = qmax
            s64[r] = s_sat
            b64[r] = -s_sat * qmax       # exact in fp16 and bf16: qmax * 2^-e, qmax < 2^8
    p.codes = codes
    p.scales = _round(s64, dtype)
    p.biases = _round(b64, dtype)
    x64 = rng.standard_normal(size=(M, K))
    big = 60000.0 * np.sign(rng.standard_normal(size=(M, K))) * rng.uniform(0.5, 1.0, size=(M, K))
    for m, kind in enumerate(row_kinds):
        if kind == "zero":
            x64[m] = 0.0
        elif kind == "large":
            x64[m] = big[m]
    p.x = _round(x64, dtype)
    return p


def check(y, dp, label):
    ref, absum = dp.oracle()
    ratio = _gpu.assert_parity(y, ref, absum, label)
    print(f"{label}: max err/bound {ratio:.3g}")
    yn = y.detach().cpu().numpy()
    # zero-weight rows and zero activation rows are exact zeros
    for r in ZERO_ROWS:
        assert np.all(yn[:, r] == 0.0), f"{label}: zero-weight row {r} not exactly 0: {yn[:, r]}"
    for m in range(yn.shape[0]):
        if not np.any(dp.p.x[m]):
            assert np.all(yn[m] == 0.0), f"{label}: zero activation row {m} not exactly 0"
    return ratio


X_CASES = [(1, "random"), (1, "zero"), (1, "large"), (3, "mixed"), (16, "mixed"), (3, "mixed_large"),
           (16, "mixed_large")]


@pytest.mark.parametrize("bits,G", [c[:2] for c in CASES])
@pytest.mark.parametrize("M,x_case", X_CASES)
@pytest.mark.parametrize("kernel", ["auto", "qmv", "mfma", "mfma_lds", "rowexact"])
def test_edge_forward(bits, G, M, x_case, kernel):
    p = edge_problem(bits, G, M, x_case, seed=100 + bits + M)
    dp = _gpu.DeviceProblem(p)
    qmm = _gpu.lib()
    if kernel == "auto":
        y = qmm.qmm_forward(dp.x, dp.wq, dp.s, dp.b, bits, G)
    elif kernel == "rowexact":
        y = qmm.qmm_forward_rowexact(dp.x, dp.wq, dp.s, dp.b, bits, G)
    else:
        y = qmm.qmm_forward_kernel(kernel, dp.x, dp.wq, dp.s, dp.b, bits, G)
    torch.cuda.synchronize()
    check(y, dp, f"{kernel} bits={bits} G={G} M={M} x={x_case}")


@pytest.mark.parametrize("bits,G", [c[:2] for c in CASES])
@pytest.mark.parametrize("M,x_case", X_CASES)
def test_edge_bf16(bits, G, M, x_case):
    p = edge_problem(bits, G, M, x_case, seed=200 + bits + M, dtype="bf16")
    dp = _gpu.DeviceProblem(p)
    y = _gpu.lib().qmm_forward_bf16(dp.x, dp.wq, dp.s, dp.b, bits, G)
    torch.cuda.synchronize()
    check(y, dp, f"bf16 bits={bits} G={G} M={M} x={x_case}")


@pytest.mark.parametrize("bits,G", [c[:2] for c in CASES])
@pytest.mark.parametrize("M,x_case", X_CASES)
@pytest.mark.parametrize("split", [2, 3])
def test_edge_splitk(bits, G, M, x_case, split):
    p = edge_problem(bits, G, M, x_case, seed=300 + bits + M)
    dp = _gpu.DeviceProblem(p)
    y = _gpu.lib().qmm_forward_splitk(dp.x, dp.wq, dp.s, dp.b, bits, G, split)
    torch.cuda.synchronize()
    check(y, dp, f"splitk S={split} bits={bits} G={G} M={M} x={x_case}")


@pytest.mark.parametrize("bits,G", [(4, 32), (2, 32), (8, 64)])
@pytest.mark.parametrize("M,x_case", X_CASES)
def test_edge_tiled(bits, G, M, x_case):
    p = edge_problem(bits, G, M, x_case, seed=400 + bits + M)
    dp = _gpu.DeviceProblem(p)
    qmm = _gpu.lib()
    tw, tsb = qmm.qmm_repack_tiled(dp.wq, dp.s, dp.b, bits, G)
    y = qmm.qmm_forward_tiled(dp.x, tw, tsb, N, bits, G)
    torch.cuda.synchronize()
    check(y, dp, f"tiled bits={bits} G={G} M={M} x={x_case}")


@pytest.mark.parametrize("bits,G", [(4, 32), (5, 64)])
@pytest.mark.parametrize("M,x_case", X_CASES)
def test_edge_fused(bits, G, M, x_case):
    """Two projections of one x, both with the degenerate rows."""
    p1 = edge_problem(bits, G, M, x_case, seed=500 + bits + M)
    p2 = edge_problem(bits, G, M, x_case, seed=600 + bits + M)
    p2.x = p1.x
    d1, d2 = _gpu.DeviceProblem(p1), _gpu.DeviceProblem(p2)
    y1, y2 = _gpu.lib().qmm_forward_fused(d1.x, [(d1.wq, d1.s, d1.b), (d2.wq, d2.s, d2.b)], bits, G)
    torch.cuda.synchronize()
    check(y1, d1, f"fused[0] bits={bits} M={M} x={x_case}")
    check(y2, d2, f"fused[1] bits={bits} M={M} x={x_case}")
