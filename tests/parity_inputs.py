"""Inputs for parity tests: seeded generators plus the oracle's own packing.

For the random-format workload the centroid table, packed bytes and scales
come straight from the generators.  For packed workloads the weights come
from the generators, the centroid table from tests/golden/centroids.json
(fitted by the oracle, see make_centroids.py) and the scales and packed
bytes from the oracle's frozen-centroid encoder.  Nothing here calls the
library.
"""
from __future__ import annotations

import functools
import json
import os

import numpy as np

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@functools.lru_cache(maxsize=None)
def golden_centroids():
    with open(os.path.join(GOLDEN, "centroids.json")) as f:
        return json.load(f)


def centroids_for(lin) -> np.ndarray:
    entry = golden_centroids()[f"cfg{lin.config_id}.mat{lin.matrix_id}"]
    assert entry["N"] == lin.N and entry["K"] == lin.K
    return np.array(entry["C"], np.uint8)


@functools.lru_cache(maxsize=4)
def packed_matrix(lin):
    """(C, alpha, packed) for a packed workload matrix."""
    if lin.config_id == 0:
        T = oracle.num_triples(lin.N)
        C = workloads.random_centroids(0, lin.matrix_id)
        packed = workloads.random_packed(0, T, lin.K, lin.matrix_id)
        alpha = workloads.random_scales_bf16(0, 3 * T, lin.matrix_id)
        return C, alpha, packed
    C = centroids_for(lin)
    W = workloads.weights(lin)
    alpha, packed = oracle.encode(W, C)
    return C, alpha, packed


def random_format(seed_words, N: int, K: int):
    """A random format instance for shape fuzzing: (C, alpha, packed)."""
    T = oracle.num_triples(N)
    C = workloads.uniform_centroids(list(seed_words) + [1], 0, 127)
    packed = workloads.uniform_bytes(list(seed_words) + [2], T, K)
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(seed_words) + [3])))
    alpha = oracle.f32_to_bf16(g.lognormal(-5, 0.3, size=3 * T).astype(np.float32))
    alpha[N:] = 0
    return C, alpha, packed
