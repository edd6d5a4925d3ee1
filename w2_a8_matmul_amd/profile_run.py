"""Fixed launch sequences for hardware-counter profiling (rocprofv3 --pmc).

Runs, in one process and in this order:
  1. ``copy``: a plain device-to-device copy of 256 MiB (torch ``copy_``),
     repeated 4 times; its FETCH_SIZE / WRITE_SIZE per dispatch against the
     known 256 MiB gives the counter scale factor;
  2. ``gemv_c1_m1``: s3d8_forward on the decode GEMV shape M=1, K=4096,
     N=14336, 28 distinct weight copies (so that every launch reads its
     weights from HBM, not from the Infinity Cache), 2 passes over them;
  3. ``gemm_c3``: s3d8_linear on the prefill shape M=2048, K=4096, N=14336,
     150 warm-up launches (the clocks settle under sustained load), then 4
     launches: the summaries use the last 4 dispatches;
  4. the same problem through s3d8_linear_unfused (dequant_tiled_kernel +
     gemm_i8_kernel), 4 calls;
  5. ``gemv_codes_c1_m8``: s3d8_linear at M=8 on the decode GEMV shape (the
     GEMV on INT8 codes), 28 weight copies, 2 passes;
  6. ``splitk_vision_down``: s3d8_linear_splitk on M=1601, K=5120, N=1280 at
     the library's split count, 50 warm-up launches, then 4.
Weights are random S3D8 formats (uniform bytes, random table and scales):
the bytes moved do not depend on the values.

Usage: python -m w2_a8_matmul_amd.profile_run   (from the repository root)
"""
from __future__ import annotations

import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def main() -> None:
    import numpy as np
    import torch

    import w2_a8_matmul_amd as s3d8
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def say(msg):
        print(f"[profile_run] {msg}", flush=True)

    # 1. copy kernel of known size
    nbytes = 256 * 2 ** 20
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).random_(0, 255)
    dst = torch.empty_like(src)
    for _ in range(4):
        dst.copy_(src)
    torch.cuda.synchronize()
    say(f"copy: 4 x {nbytes} bytes")
    del src, dst

    def fmt(seed, N, K):
        T = s3d8.num_triples(N)
        C = torch.from_numpy(workloads.random_centroids(seed)).to(dev)
        S = torch.from_numpy(workloads.random_scales_bf16(seed, 3 * T).view(np.int16)).to(dev)
        P = torch.from_numpy(workloads.random_packed(seed, T, K)).to(dev)
        return C, S, s3d8.tile(P, N)

    # 2. decode GEMV, fused forward
    M, K, N = 1, 4096, 14336
    C, S, tiled = fmt(11, N, K)
    copies = [tiled.clone() for _ in range(28)]
    x = torch.randn((M, K), dtype=torch.float32, device=dev)
    y = torch.empty((M, N), dtype=torch.float32, device=dev)
    xq = torch.empty((M, K), dtype=torch.int8, device=dev)
    xs = torch.empty((M,), dtype=torch.float32, device=dev)
    for _ in range(2):
        for t in copies:
            s3d8.forward(x, t, C, S, N, y=y, xq=xq, xs=xs)
    torch.cuda.synchronize()
    say(f"gemv_c1_m1: {2 * len(copies)} launches of s3d8_forward M={M} K={K} N={N}")
    del copies, tiled

    # 3. prefill GEMM
    M = 2048
    C, S, tiled = fmt(12, N, K)
    x = torch.randn((M, K), dtype=torch.float32, device=dev)
    xq, xs = s3d8.quant_act(x)
    y = torch.empty((M, N), dtype=torch.float32, device=dev)
    for _ in range(150 + 4):
        s3d8.linear(xq, xs, tiled, C, S, N, y=y)
    torch.cuda.synchronize()
    say(f"gemm_c3: 150 + 4 launches of s3d8_linear M={M} K={K} N={N}")

    # 4. the unfused prefill path on the same problem
    ws = torch.empty((s3d8.unfused_workspace_bytes(N, K),), dtype=torch.int8, device=dev)
    for _ in range(4):
        s3d8.linear_unfused(xq, xs, tiled, C, S, N, workspace=ws, y=y)
    torch.cuda.synchronize()
    say(f"gemm_c3 unfused: 4 calls of s3d8_linear_unfused M={M} K={K} N={N}")
    del ws, tiled, y

    # 5. the GEMV on INT8 codes, eight tokens
    M = 8
    C, S, tiled = fmt(13, N, K)
    copies = [tiled.clone() for _ in range(28)]
    xq, xs = s3d8.quant_act(torch.randn((M, K), dtype=torch.float32, device=dev))
    y = torch.empty((M, N), dtype=torch.float32, device=dev)
    for _ in range(2):
        for t in copies:
            s3d8.linear(xq, xs, t, C, S, N, y=y)
    torch.cuda.synchronize()
    say(f"gemv_codes_c1_m8: {2 * len(copies)} launches of s3d8_linear M={M} K={K} N={N}")
    del copies, tiled

    # 6. split-K on the vision down-projection
    M, K, N = 1601, 5120, 1280
    C, S, tiled = fmt(14, N, K)
    xq, xs = s3d8.quant_act(torch.randn((M, K), dtype=torch.float32, device=dev))
    y = torch.empty((M, N), dtype=torch.float32, device=dev)
    splits = s3d8.splitk_auto(M, K, N, torch.cuda.get_device_properties(dev).multi_processor_count)
    wsk = torch.zeros((max(1, s3d8.splitk_workspace_bytes(M, K, N, splits)),), dtype=torch.uint8, device=dev)
    for _ in range(50 + 4):
        s3d8.linear_splitk(xq, xs, tiled, C, S, N, splits=splits, workspace=wsk, y=y)
    torch.cuda.synchronize()
    say(f"splitk_vision_down: 50 + 4 launches of s3d8_linear_splitk M={M} K={K} N={N} splits={splits}")


if __name__ == "__main__":
    main()
