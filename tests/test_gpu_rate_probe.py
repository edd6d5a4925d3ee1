"""The measurement probes the bench reads the kernels against.

Matrix-core rate probe (the GEMM's ceiling): every output word must equal
2048 v^2 iters (mod 2^32), the value four chains of 32 x 32 x 32 INT8
products over bytes all equal to v accumulate, so a probe that skipped or
merged its products would not pass.

Memory read probe (the GEMV's ceiling at the same transfer size): each
workgroup's word must be the XOR of exactly the words it is defined to read,
so a probe that skipped loads would not pass."""
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


@pytest.mark.parametrize("nbytes,wgs", [(16, 1), (4096, 3), (19_603_552, 1024), (1 << 20, 7)])
def test_hbm_read_probe_xor(gpu, nbytes, wgs):
    """Workgroup w stores the XOR of the 32-bit words of the 16-byte chunks c
    with (c / 256) % wgs == w; the XOR over workgroups is the XOR of the whole
    buffer."""
    g = np.random.Generator(np.random.PCG64([5000, nbytes]))
    words = g.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(words.view(np.int32).copy()).to(gpu)
    out = s3d8.hbm_read_probe(buf, wgs)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint32)
    chunk_words = words.reshape(-1, 4)
    owner = (np.arange(chunk_words.shape[0]) // 256) % wgs
    ref = np.zeros(wgs, np.uint32)
    for w in range(wgs):
        sel = chunk_words[owner == w]
        ref[w] = np.bitwise_xor.reduce(sel.reshape(-1)) if sel.size else 0
    np.testing.assert_array_equal(got, ref)
    assert np.bitwise_xor.reduce(got) == np.bitwise_xor.reduce(words)
