"""The matrix-core rate probe that the bench reads the GEMM against: every
output word must equal 2048 v^2 iters (mod 2^32), the value four chains of
32 x 32 x 32 INT8 products over bytes all equal to v accumulate, so a probe
that skipped or merged its products would not pass."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
s3d8 = pytest.importorskip("w2_a8_matmul_amd")


@pytest.mark.parametrize("iters,workgroups,v", [(1, 1, 1), (3, 8, 5), (7, 300, -3), (100, 16, -128), (2, 4, 0)])
def test_rate_probe_value(gpu, iters, workgroups, v):
    out, ops = s3d8.mfma_rate_probe(iters, workgroups, v, device=gpu)
    torch.cuda.synchronize()
    want = np.array([(2048 * v * v * iters) % 2 ** 32], np.uint32).view(np.int32)[0]
    got = out.cpu().numpy()
    assert got.shape == (256 * workgroups,)
    assert (got == want).all(), (int(want), np.unique(got)[:4])
    assert ops == workgroups * 16 * iters * 65536


def test_rate_probe_rejects_short_output(gpu):
    out = torch.empty((255,), dtype=torch.int32, device=gpu)
    with pytest.raises(ValueError):
        s3d8.mfma_rate_probe(1, 1, 1, out=out)
