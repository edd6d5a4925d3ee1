"""Write tests/golden/centroids.json: the centroid table of every packed
workload matrix, fitted by the ORACLE (oracle.fit_centroids: k-means++ and
Lloyd-Max as in "Llama-Mobile: Efficient 2.7-Bit Quantization of VLMs",
Sec. 3.4) on that matrix's seeded synthetic weights.

The GPU parity tests then take these tables, encode the weights with the
oracle's frozen-centroid encoder, and feed the same bytes to the library and
the oracle, so no oracle input comes from the library.

Calls only oracle/ and the seeded generators.  Usage:
    python tests/golden/make_centroids.py [name ...]
"""
from __future__ import annotations

import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads  # noqa: E402

OUT = os.path.join(HERE, "centroids.json")
MAX_ITERS = 10


def matrices():
    seen = {}
    for lin in [workloads.C1[1], *workloads.C2, workloads.C3, *workloads.C4]:
        key = (lin.config_id, lin.matrix_id)
        if key not in seen:
            seen[key] = lin
    return list(seen.values())


def key_of(lin) -> str:
    return f"cfg{lin.config_id}.mat{lin.matrix_id}"


def main(names):
    data = {}
    if os.path.exists(OUT):
        with open(OUT) as f:
            data = json.load(f)
    for lin in matrices():
        k = key_of(lin)
        if names and k not in names:
            continue
        t0 = time.time()
        W = workloads.weights(lin)
        C, cent, dist, it = oracle.fit_centroids(W, lin.pack_seed, MAX_ITERS)
        data[k] = {
            "matrix": lin.name, "config_id": lin.config_id, "matrix_id": lin.matrix_id,
            "N": lin.N, "K": lin.K, "seed": lin.pack_seed, "max_iters": MAX_ITERS,
            "iterations": it, "distortion_first": float(dist[0]), "distortion_last": float(dist[-1]),
            "C": C.tolist(),
        }
        print(f"{k} {lin.name} N={lin.N} K={lin.K} iters={it} {time.time() - t0:.1f}s", flush=True)
        del W
        with open(OUT, "w") as f:
            json.dump(data, f, indent=1, sort_keys=True)


if __name__ == "__main__":
    main(sys.argv[1:])
