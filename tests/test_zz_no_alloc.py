"""s3d8_linear_unfused_noalloc, the entry point for callers that cannot
allocate device memory, against s3d8_linear_unfused with a workspace (the
entry point it is a variant of), through the C ABI.

Two calls in a row on one GPU share the library's device scratch array: the
first decodes a c1-shaped matrix (K = 4096, N = 14336: 58.8 MB decoded, near
the 64 MiB limit), the second a smaller one, which must not see anything of
the first.  Accumulators and outputs must be identical to the workspace path
and to the oracle on the smaller call.  A matrix whose decoded size exceeds
the scratch is refused before any launch.
"""
import ctypes

import numpy as np
import pytest

import oracle
import workloads
from parity_inputs import random_format

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
s3d8 = pytest.importorskip("w2_a8_matmul_amd")
from w2_a8_matmul_amd import _lib  # noqa: E402


def _dev(a, gpu):
    return torch.from_numpy(np.ascontiguousarray(a)).to(gpu)


def _noalloc(xq, xs, tiled, C, S, N, y, acc):
    M, K = xq.shape
    _lib.call("s3d8_linear_unfused_noalloc", xq.data_ptr(), xs.data_ptr(), M, K, N, tiled.data_ptr(), tiled.numel(),
              C.data_ptr(), S.data_ptr(), y.data_ptr(), acc.data_ptr() if acc is not None else None,
              torch.cuda.current_stream(xq.device).cuda_stream)


def _case(gpu, M, K, N, seed):
    C, alpha, packed = random_format([seed, M, K, N], N, K)
    x = workloads.gaussian_matrix([seed + 1, M, K], M, K)
    xq, xs = s3d8.quant_act(_dev(x, gpu))
    tiled = s3d8.tile(_dev(packed, gpu), N)
    return x, C, alpha, packed, xq, xs, tiled, _dev(C, gpu), _dev(alpha.view(np.int16), gpu)


def test_noalloc_matches_workspace_path_two_calls(gpu):
    assert s3d8.unfused_workspace_bytes(14336, 4096) <= _lib.S3D8_NOALLOC_SCRATCH_BYTES
    results = []
    for (M, K, N, seed) in [(320, 4096, 14336, 6000), (40, 1040, 97, 6010)]:
        x, C, alpha, packed, xq, xs, tiled, dC, dS = _case(gpu, M, K, N, seed)
        y_na = torch.full((M, N), float("nan"), dtype=torch.float32, device=gpu)
        acc_na = torch.full((M, N), -1, dtype=torch.int32, device=gpu)
        _noalloc(xq, xs, tiled, dC, dS, N, y_na, acc_na)
        y_ws, acc_ws = s3d8.linear_unfused(xq, xs, tiled, dC, dS, N, return_acc=True)
        y_only = torch.full((M, N), float("nan"), dtype=torch.float32, device=gpu)
        _noalloc(xq, xs, tiled, dC, dS, N, y_only, None)  # the accumulator-free kernel build
        torch.cuda.synchronize()
        np.testing.assert_array_equal(acc_na.cpu().numpy(), acc_ws.cpu().numpy())
        np.testing.assert_array_equal(y_na.cpu().numpy(), y_ws.cpu().numpy())
        np.testing.assert_array_equal(y_only.cpu().numpy(), y_ws.cpu().numpy())
        results.append((x, C, alpha, packed, N, acc_na.cpu().numpy(), y_na.cpu().numpy()))
    # the second, smaller call against the oracle as well
    x, C, alpha, packed, N, acc, y = results[1]
    _, _, acc_r, y_r = oracle.linear(x, packed, C, alpha, N)
    np.testing.assert_array_equal(acc, acc_r)
    np.testing.assert_array_equal(y, y_r)


def test_noalloc_refuses_matrix_over_scratch(gpu):
    """The vocabulary projection (K = 4096, N = 128256) decodes to 525 MB:
    SHAPE, and nothing is written."""
    K, N, M = 4096, 128256, 17
    assert s3d8.unfused_workspace_bytes(N, K) > _lib.S3D8_NOALLOC_SCRATCH_BYTES
    xq = torch.zeros((M, K), dtype=torch.int8, device=gpu)
    xs = torch.zeros((M,), dtype=torch.float32, device=gpu)
    tiled = torch.zeros((s3d8.tiled_bytes(N, K),), dtype=torch.uint8, device=gpu)
    C = torch.zeros((96,), dtype=torch.uint8, device=gpu)
    S = torch.zeros((N + 2,), dtype=torch.int16, device=gpu)
    y = torch.full((M, N), 7.0, dtype=torch.float32, device=gpu)
    with pytest.raises(s3d8.S3D8Error) as e:
        _noalloc(xq, xs, tiled, C, S, N, y, None)
    assert e.value.code == _lib.S3D8_ERR_SHAPE and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert (y == 7.0).all().item()
