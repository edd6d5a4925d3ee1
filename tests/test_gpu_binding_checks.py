"""The Python binding refuses caller-supplied buffers of the wrong type, size
or device before anything is queued, so a kernel never writes past a
caller's buffer (e.g. an fp32 output into a bf16 tensor of half the bytes)."""
import numpy as np
import pytest

import workloads
from parity_inputs import random_format

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
s3d8 = pytest.importorskip("w2_a8_matmul_amd")


def _inputs(gpu, M=3, K=64, N=10):
    C, alpha, packed = random_format([4100, M, K, N], N, K)
    x = torch.from_numpy(workloads.gaussian_matrix([4101], M, K)).to(gpu)
    tiled = s3d8.tile(torch.from_numpy(packed).to(gpu), N)
    return x, tiled, torch.from_numpy(C).to(gpu), torch.from_numpy(alpha.view(np.int16)).to(gpu), M, K, N


def test_linear_rejects_bad_outputs(gpu):
    x, tiled, C, S, M, K, N = _inputs(gpu)
    xq, xs = s3d8.quant_act(x)
    with pytest.raises(TypeError):  # fp32 output asked, bf16 buffer given
        s3d8.linear(xq, xs, tiled, C, S, N, y=torch.empty((M, N), dtype=torch.bfloat16, device=gpu))
    with pytest.raises(TypeError):  # bf16 output asked, fp32 buffer given
        s3d8.linear(xq, xs, tiled, C, S, N, y=torch.empty((M, N), dtype=torch.float32, device=gpu), out="bf16")
    with pytest.raises(ValueError):
        s3d8.linear(xq, xs, tiled, C, S, N, y=torch.empty((M, N - 1), dtype=torch.float32, device=gpu))
    with pytest.raises(ValueError):
        s3d8.linear(xq, xs, tiled, C, S, N, acc=torch.empty((M - 1, N), dtype=torch.int32, device=gpu),
                    return_acc=True)
    with pytest.raises(ValueError):
        s3d8.linear(xq, xs[: M - 1], tiled, C, S, N)
    with pytest.raises(ValueError):  # tiled buffer too small for (N, K)
        s3d8.linear(xq, xs, tiled[:-1], C, S, N)
    with pytest.raises(ValueError):
        s3d8.linear_unfused(xq, xs, tiled, C, S, N, y=torch.empty((M * N + 1,), dtype=torch.float32, device=gpu))
    with pytest.raises(ValueError):
        s3d8.linear_unfused(xq, xs, tiled, C, S, N,
                            workspace=torch.empty((16,), dtype=torch.int8, device=gpu))
    torch.cuda.synchronize()


def test_forward_rejects_bad_outputs(gpu):
    x, tiled, C, S, M, K, N = _inputs(gpu)
    with pytest.raises(ValueError):
        s3d8.forward(x, tiled, C, S, N, xq=torch.empty((M, K - 16), dtype=torch.int8, device=gpu))
    with pytest.raises(ValueError):
        s3d8.forward(x, tiled, C, S, N, xs=torch.empty((M + 1,), dtype=torch.float32, device=gpu))
    with pytest.raises(TypeError):
        s3d8.forward(x, tiled, C, S, N, xs=torch.empty((M,), dtype=torch.float64, device=gpu))
    with pytest.raises(TypeError):
        s3d8.forward(x, tiled, C, S, N, y=torch.empty((M, N), dtype=torch.float32))  # host tensor
    with pytest.raises(ValueError):
        s3d8.forward_batch([dict(x=x, tiled=tiled, centroids=C, scales=S, N=N,
                                 y=torch.empty((M, N + 3), dtype=torch.float32, device=gpu))])
    with pytest.raises(ValueError):
        s3d8.quant_act(x, xq=torch.empty((M * K - 1,), dtype=torch.int8, device=gpu))
    with pytest.raises(ValueError):
        s3d8.dequant(torch.zeros((4, K), dtype=torch.uint8, device=gpu), C, N,
                     w=torch.empty((N, K - 16), dtype=torch.int8, device=gpu))
    torch.cuda.synchronize()


def test_accepted_buffers_still_work(gpu):
    """The same calls with correctly sized buffers run (the checks refuse
    only what does not fit)."""
    x, tiled, C, S, M, K, N = _inputs(gpu)
    y = torch.empty((M * N,), dtype=torch.float32, device=gpu)  # any shape with M * N elements
    xq = torch.empty((M, K), dtype=torch.int8, device=gpu)
    xs = torch.empty((M,), dtype=torch.float32, device=gpu)
    s3d8.forward(x, tiled, C, S, N, y=y, xq=xq, xs=xs)
    y2 = s3d8.linear(xq, xs, tiled, C, S, N)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(y.view(M, N).cpu().numpy(), y2.cpu().numpy())
