"""Seeded synthetic inputs for the affine group-quantized matrix product.

This module only draws random numbers. It holds none of the product's
arithmetic (no packing, no dequantization, no dot products), so both the
CPU oracle and the GPU library can be fed from it without sharing any of
the computation.

Every tensor comes from numpy's PCG64 generator (``numpy.random.default_rng``)
and is drawn in a fixed order: codes (or packed words), scales, biases, x.
Values are drawn in float64 and rounded once to float16 (round to nearest
even, numpy's ``astype``). For bfloat16 operands (``dtype="bf16"``) the same
draws are rounded to float32 and then to bfloat16, both to nearest even,
and kept as uint16 bit patterns (numpy has no bfloat16 type).

Distributions (the workloads described for the verify-block projections in
the vmlx-swift pull request #565 page, commit "LaneQMM", and the
"Qwen3.8 Flash Next performance and parity receipt" page, section
"MTPLX logic review", which lists the 4-bit/group-32, 4-bit/group-64 and
8-bit formats consumed as stored):

* codes   : uniform integers over the full range 0 .. 2**bits - 1
* scales  : U(0.005, 0.02), rounded to fp16
* biases  : U(-0.1, 0.1), rounded to fp16
* x       : N(0, 1), rounded to fp16

Rows of the packed matrix are a whole number of 32-bit words whenever
32 divides K, so uniformly random uint32 words are exactly i.i.d. uniform
codes; ``packed_words=True`` draws the words directly (used for the large
workloads, where drawing 89 M codes and packing them on the host would be
slow).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

SCALE_RANGE = (0.005, 0.02)
BIAS_RANGE = (-0.1, 0.1)


def rng_for(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


def draw_codes(rng: np.random.Generator, N: int, K: int, bits: int) -> np.ndarray:
    """uint8 [N, K], uniform over 0 .. 2**bits - 1."""
    return rng.integers(0, 1 << bits, size=(N, K), dtype=np.uint8)


def draw_words(rng: np.random.Generator, N: int, K: int, bits: int) -> np.ndarray:
    """uint32 [N, K*bits/32] of uniform random words (requires 32 | K*bits)."""
    if (K * bits) % 32:
        raise ValueError("K*bits must be a multiple of 32 to draw whole words")
    return rng.integers(0, 1 << 32, size=(N, K * bits // 32), dtype=np.uint32)


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float64 -> float32 -> bfloat16 (each to nearest even), as uint16 bit
    patterns. Inputs are finite and far from the float32 limits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def _round(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f16":
        return a.astype(np.float16)
    if dtype == "bf16":
        return to_bf16_bits(a)
    raise ValueError("dtype must be 'f16' or 'bf16'")


def draw_scales(rng: np.random.Generator, N: int, Kg: int, dtype: str = "f16") -> np.ndarray:
    return _round(rng.uniform(*SCALE_RANGE, size=(N, Kg)), dtype)


def draw_biases(rng: np.random.Generator, N: int, Kg: int, dtype: str = "f16") -> np.ndarray:
    return _round(rng.uniform(*BIAS_RANGE, size=(N, Kg)), dtype)


def draw_x(rng: np.random.Generator, M: int, K: int, dtype: str = "f16") -> np.ndarray:
    return _round(rng.standard_normal(size=(M, K)), dtype)


@dataclass
class Problem:
    """One seeded problem instance. Exactly one of ``codes``/``words`` is set."""

    M: int
    K: int
    N: int
    bits: int
    G: int
    seed: int
    x: np.ndarray
    scales: np.ndarray
    biases: np.ndarray
    codes: np.ndarray | None = None
    words: np.ndarray | None = None
    dtype: str = "f16"  # type of x, scales and biases: "f16" or "bf16" (uint16 bit patterns)
    meta: dict = field(default_factory=dict)


def make_problem(seed: int, M: int, K: int, N: int, bits: int, G: int,
                 packed_words: bool = False, dtype: str = "f16") -> Problem:
    if K % G:
        raise ValueError("K must be a multiple of G")
    rng = rng_for(seed)
    codes = words = None
    if packed_words:
        words = draw_words(rng, N, K, bits)
    else:
        codes = draw_codes(rng, N, K, bits)
    Kg = K // G
    scales = draw_scales(rng, N, Kg, dtype)
    biases = draw_biases(rng, N, Kg, dtype)
    x = draw_x(rng, M, K, dtype)
    return Problem(M=M, K=K, N=N, bits=bits, G=G, seed=seed, x=x,
                   scales=scales, biases=biases, codes=codes, words=words, dtype=dtype)
