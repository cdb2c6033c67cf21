"""Seeded synthetic workloads for the EQ-Linear hot path.

This module holds shapes, seeds and random draws only -- none of the layer's
arithmetic.  Both the parity tests (which feed the float64 oracle) and the
benchmark draw their inputs here, so both sides see identical values.

Shapes follow the operator benchmarks and the ViT-style layer shapes of the
pages ([pchao] §4.1: B=32, L=1024, T=4, C_T up to 2048, D=C; the ViT/Swin
study of [pchao] §4.2 at 224x224 with 16x16 patches gives 197 tokens per
image).  The pages measure on ImageNet-100 with trained networks; seeded
Gaussians stand in for those activations and weights (kernel time does not
depend on the values).

Recipe: numpy PCG64 ``default_rng(seed)``; draw in float64, scale, then cast
to the run dtype with round-to-nearest-even.  X ~ N(0,1) [N,C_T,T],
Wt ~ N(0, 1/C_in) [D_T,C_T,T] with C_in = C_T*T of that layer, dY ~ N(0,1)
[N,D_T,T], and, where a bias is used, b ~ N(0,1) [D_T].
Seed = 1000*cfg + 10*sub + {0: X, 1: Wt, 2: dY, 3: b}.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str        # short identifier used by tests and the benchmark
    cfg: int         # configuration number (seed base)
    sub: int         # variant inside the configuration (seed offset)
    N: int           # rows = batch x tokens
    C_T: int         # input channels per group element
    D_T: int         # output channels per group element
    T: int           # group order (components per tuple)
    dtypes: tuple    # I/O dtypes it is run in
    backward: bool   # whether the gradients are part of the workload
    what: str        # plain description

    @property
    def C(self) -> int:
        return self.C_T * self.T

    @property
    def D(self) -> int:
        return self.D_T * self.T

    def seed(self, which: int) -> int:
        return 1000 * self.cfg + 10 * self.sub + which


WORKLOADS = {
    w.name: w
    for w in [
        Workload("p4_tiny", 1, 0, 64, 16, 16, 4, ("f32",), False,
                 "p4, N=64, C=64 -> D=64, forward only"),
        Workload("vits_qkv", 2, 0, 64 * 197, 96, 288, 4, ("f32", "f16"), True,
                 "ViT-S-like attention qkv projection, N=64x197, C=384 -> D=1152"),
        Workload("vits_proj", 2, 1, 64 * 197, 96, 96, 4, ("f32", "f16"), True,
                 "ViT-S-like attention output projection, N=64x197, C=384 -> D=384"),
        Workload("vitb_fc1", 3, 0, 64 * 197, 192, 768, 4, ("f16",), True,
                 "ViT-B-like FFN fc1, N=64x197, C=768 -> D=3072"),
        Workload("vitb_fc2", 3, 1, 64 * 197, 768, 192, 4, ("f16",), True,
                 "ViT-B-like FFN fc2, N=64x197, C=3072 -> D=768"),
        Workload("square4096", 4, 0, 32768, 1024, 1024, 4, ("f16",), True,
                 "compute-bound square layer, N=32768, C=D=4096"),
        Workload("square4096_n256", 4, 1, 256, 1024, 1024, 4, ("f16",), True,
                 "memory-bound square layer, N=256, C=D=4096"),
        Workload("c8_wide", 5, 0, 16384, 128, 512, 8, ("f32", "f16"), True,
                 "cyclic group C8, N=16384, C=1024 -> D=4096"),
        Workload("c3_vitb_fc1", 6, 0, 64 * 197, 256, 1024, 3, ("f16",), True,
                 "cyclic group C3 at ViT-B FFN fc1 size, N=64x197, C=768 -> D=3072"),
        Workload("c6_vitb_fc1", 6, 1, 64 * 197, 128, 512, 6, ("f32", "f16"), True,
                 "cyclic group C6 at ViT-B FFN fc1 size, N=64x197, C=768 -> D=3072"),
    ]
}

# Layers over the octic group D8 (quarter turns and reflections, T = 8
# components per tuple; the group of the isotypic-basis ViTs that [paperpeel]
# App. A.2 and A.4 compare against), at the same layer sizes as the cyclic
# ones above.
OCTIC_WORKLOADS = {
    w.name: w
    for w in [
        Workload("d8_vitb_fc1", 7, 0, 64 * 197, 96, 384, 8, ("f32", "f16"), True,
                 "octic group D8 at ViT-B FFN fc1 size, N=64x197, C=768 -> D=3072"),
        Workload("d8_wide", 7, 1, 16384, 128, 512, 8, ("f32", "f16"), True,
                 "octic group D8, N=16384, C=1024 -> D=4096"),
    ]
}

# The group-size scaling of the operator benchmark ([paperpeel] App. A.4,
# "Scaling with the group size": T = 2, 4, 8 at C/T = 2048 channels per
# group element, the batch of [pchao] §4.1, B = 32 x L = 1024 rows), square
# layers.
SCALING_WORKLOADS = {
    w.name: w
    for w in [
        Workload("tscale_t2", 8, 0, 32 * 1024, 2048, 2048, 2, ("f16",), True,
                 "group-size scaling, T=2, N=32768, C=D=4096 (C/T=2048)"),
        Workload("tscale_t4", 8, 1, 32 * 1024, 2048, 2048, 4, ("f16",), True,
                 "group-size scaling, T=4, N=32768, C=D=8192 (C/T=2048)"),
        Workload("tscale_t8", 8, 2, 32 * 1024, 2048, 2048, 8, ("f16",), True,
                 "group-size scaling, T=8, N=32768, C=D=16384 (C/T=2048)"),
    ]
}

# The workload the headline metric is quoted on.
HEADLINE = "vitb_fc1"

NP_DTYPE = {"f32": np.float32, "f16": np.float16}


def draw(shape, seed: int, std: float, dtype: str) -> np.ndarray:
    """Seeded N(0, std^2) draw, float64 then rounded to ``dtype``."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal(size=shape, dtype=np.float64)
    if std != 1.0:
        a *= std
    return a.astype(NP_DTYPE[dtype])


def inputs(w: Workload, dtype: str, N: int | None = None):
    """(X, Wt, dY) for workload ``w`` in ``dtype``; N overrides the row count."""
    n = w.N if N is None else N
    x = draw((n, w.C_T, w.T), w.seed(0), 1.0, dtype)
    wt = draw((w.D_T, w.C_T, w.T), w.seed(1), (1.0 / w.C) ** 0.5, dtype)
    dy = draw((n, w.D_T, w.T), w.seed(2), 1.0, dtype)
    return x, wt, dy


def bias_input(D_T: int, dtype: str, seed: int) -> np.ndarray:
    """Group-shared bias b [D_T] ~ N(0, 1) (seed: the workload's seed(3))."""
    return draw((D_T,), seed, 1.0, dtype)


def custom_inputs(N, C_T, D_T, T, dtype, seed):
    """(X, Wt, dY) for an arbitrary shape, same recipe, seeds seed+{0,1,2}."""
    x = draw((N, C_T, T), seed, 1.0, dtype)
    wt = draw((D_T, C_T, T), seed + 1, (1.0 / max(1, C_T * T)) ** 0.5, dtype)
    dy = draw((N, D_T, T), seed + 2, 1.0, dtype)
    return x, wt, dy
