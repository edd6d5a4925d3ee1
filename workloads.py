"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no arithmetic of the method: it only draws random numbers
with the shapes and distributions of the workloads (Llama-3.2-11B-Vision
linear shapes from the blog's microbenchmark tables and Table 2 of the paper)
and hands them, unchanged, to both the oracle and the library.

Every tensor comes from numpy's PCG64 seeded with
``SeedSequence([config_id, tensor_id, matrix_id])``, so any tensor can be
regenerated on its own on any machine.

The real checkpoint, calibration data and benchmark datasets are not
available; these synthetic tensors stand in for them.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

# tensor ids
T_WEIGHT = 0
T_ACT = 1
T_CENTROIDS = 2
T_SCALES = 3
T_PACKED = 4


def rng(config_id: int, tensor_id: int, matrix_id: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([config_id, tensor_id, matrix_id])))


@dataclass(frozen=True)
class Linear:
    """One linear layer Y = X W^T with X [M][K], W [N][K]."""
    name: str
    config_id: int
    matrix_id: int
    M: int
    K: int
    N: int
    outliers: bool = False

    @property
    def pack_seed(self) -> int:
        return 1 + self.matrix_id


# Config 0: one small linear with a random format (no packer).
C0 = Linear("c0.small", 0, 0, 1, 256, 384)

# Config 1: text MLP gate/up shape at decode batch sizes.
C1 = {m: Linear(f"c1.mlp_up.m{m}", 1, 0, m, 4096, 14336) for m in (1, 4, 8)}

# Config 2: one decoder layer at M=1, activations with 1% outliers x20.
C2 = [
    Linear("c2.attn_q", 2, 0, 1, 4096, 4096, True),
    Linear("c2.attn_k", 2, 1, 1, 4096, 1024, True),
    Linear("c2.attn_v", 2, 2, 1, 4096, 1024, True),
    Linear("c2.attn_o", 2, 3, 1, 4096, 4096, True),
    Linear("c2.mlp_gate", 2, 4, 1, 4096, 14336, True),
    Linear("c2.mlp_up", 2, 5, 1, 4096, 14336, True),
    Linear("c2.mlp_down", 2, 6, 1, 14336, 4096, True),
]

# Config 3: prefill GEMM.
C3 = Linear("c3.prefill_mlp_up", 3, 0, 2048, 4096, 14336)

# Config 4: vocabulary projection and vision-encoder MLP.
C4 = [
    Linear("c4.lm_head.m1", 4, 0, 1, 4096, 128256),
    Linear("c4.lm_head.m512", 4, 0, 512, 4096, 128256),
    Linear("c4.vision_up", 4, 1, 1601, 1280, 5120),
    Linear("c4.vision_down", 4, 2, 1601, 5120, 1280),
]


def weights(lin: Linear) -> np.ndarray:
    """fp32 [N][K] ~ N(0, 0.02)."""
    g = rng(lin.config_id, T_WEIGHT, lin.matrix_id)
    W = g.standard_normal((lin.N, lin.K), dtype=np.float32)
    W *= np.float32(0.02)
    return W


def activations(lin: Linear, M: int | None = None) -> np.ndarray:
    """fp32 [M][K] ~ N(0,1); with ``outliers`` each element is independently
    (probability 0.01) multiplied by 20."""
    M = lin.M if M is None else M
    g = rng(lin.config_id, T_ACT, lin.matrix_id)
    x = g.standard_normal((M, lin.K), dtype=np.float32)
    if lin.outliers:
        mask = g.random((M, lin.K)) < 0.01
        x = np.where(mask, x * np.float32(20.0), x).astype(np.float32)
    return x


def random_centroids(config_id: int, matrix_id: int = 0) -> np.ndarray:
    """uint8 [32][3], uniform integers in [1, 127]."""
    return rng(config_id, T_CENTROIDS, matrix_id).integers(1, 128, size=(32, 3), dtype=np.uint8)


def random_packed(config_id: int, rows: int, K: int, matrix_id: int = 0) -> np.ndarray:
    """uint8 [rows][K], uniform over all 256 byte values.  Uniform bytes give a
    uniform 5-bit index and three independent fair sign selectors."""
    return rng(config_id, T_PACKED, matrix_id).integers(0, 256, size=(rows, K), dtype=np.uint8)


def random_scales_bf16(config_id: int, count: int, matrix_id: int = 0) -> np.ndarray:
    """bf16 bit patterns (uint16) of lognormal(mu=-5, sigma=0.3) draws,
    converted by torch's float32 -> bfloat16 cast (round to nearest even)."""
    import torch

    f = rng(config_id, T_SCALES, matrix_id).lognormal(-5.0, 0.3, size=count).astype(np.float32)
    return torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def gaussian_matrix(seed_words, rows: int, cols: int, std: float = 1.0) -> np.ndarray:
    """Generic fp32 Gaussian matrix for test shapes outside the named configs."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(seed_words))))
    return (g.standard_normal((rows, cols), dtype=np.float32) * np.float32(std)).astype(np.float32)


def uniform_bytes(seed_words, rows: int, cols: int) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(seed_words))))
    return g.integers(0, 256, size=(rows, cols), dtype=np.uint8)


def uniform_centroids(seed_words, lo: int = 1, hi: int = 127) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(seed_words))))
    return g.integers(lo, hi + 1, size=(32, 3), dtype=np.uint8)


def signed_table(seed_words, lo: int = -127, hi: int = 127) -> np.ndarray:
    """int8 [256][3], uniform integers in [lo, hi]: a 3D8 table of signed
    centroids (one row per byte value)."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(seed_words))))
    return g.integers(lo, hi + 1, size=(256, 3)).astype(np.int8)
