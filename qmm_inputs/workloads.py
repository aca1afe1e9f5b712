"""Named synthetic workloads (shapes only; values come from ``qmm_inputs``).

The shapes stand in for the projections that the vmlx-swift pull request
#565 page times during speculative verification (27B dense MLP up and down
projections, mixed 5/6/8-bit projections, a long-K down projection split
over K, and a stack of dense decoder layers). No trained weights are used:
every tensor is drawn by ``qmm_inputs.make_problem``.
"""
from __future__ import annotations

from dataclasses import dataclass


@dataclass(frozen=True)
class Shape:
    name: str
    K: int
    N: int
    bits: int
    G: int

    @property
    def Kg(self) -> int:
        return self.K // self.G

    @property
    def weight_bytes(self) -> int:
        """Codes plus fp16 scale and fp16 bias per group: N*K*(bits/8 + 4/G)."""
        return self.N * self.K * self.bits // 8 + self.N * self.Kg * 4


# Tiny: M=1, K=N=512, 4-bit, G=32, seed 0.
TINY = Shape("tiny_512x512_w4g32", K=512, N=512, bits=4, G=32)
TINY_M = (1,)

# 27B-style dense MLP up projection, 5120 -> 17408, 4-bit, G=32.
DENSE_UP = Shape("dense_up_5120x17408_w4g32", K=5120, N=17408, bits=4, G=32)
DENSE_UP_M = (1, 2, 4, 8, 16)

# Mixed-bit projections, 5120 -> 5120, G=64.
MIXED = tuple(Shape(f"mixed_5120x5120_w{b}g64", K=5120, N=5120, bits=b, G=64) for b in (5, 6, 8))
MIXED_M = (1, 8, 16)

# Long-K down projection, 17408 -> 5120, 4-bit, G=32, M=16, split over K.
LONG_K = Shape("long_k_17408x5120_w4g32", K=17408, N=5120, bits=4, G=32)
LONG_K_M = 16
LONG_K_SPLITS = (1, 2, 4, 8)

# Dense decoder layer: (name, K, N) per projection, 4-bit G=32.
LAYER_PROJECTIONS = (
    ("q", 5120, 6144),
    ("k", 5120, 1024),
    ("v", 5120, 1024),
    ("o", 6144, 5120),
    ("gate", 5120, 17408),
    ("up", 5120, 17408),
    ("down", 17408, 5120),
)
SWEEP_LAYERS = 64
SWEEP_M = (1, 8)


def sweep_shapes(layers: int = SWEEP_LAYERS):
    """Yield (layer, proj_index, Shape, seed) for the layer-stack sweep.

    Seed per matrix = 1000*layer + proj_index; layers are independent.
    """
    for layer in range(layers):
        for j, (pname, K, N) in enumerate(LAYER_PROJECTIONS):
            yield layer, j, Shape(f"L{layer}.{pname}", K=K, N=N, bits=4, G=32), 1000 * layer + j


def sweep_x_seed(layer: int, key: int, M: int) -> int:
    """Seed of the M-row input `key` of a sweep layer (0: q/k/v, 1: o,
    2: gate/up, 3: down; q/k/v and gate/up share their input)."""
    return 500_000 + 100 * layer + 10 * key + M


def sweep_weight_bytes(layers: int = SWEEP_LAYERS) -> int:
    return sum(s.weight_bytes for _, _, s, _ in sweep_shapes(layers))
