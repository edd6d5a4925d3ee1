"""GPU parity at the full prefill sizes, every output against the oracle.

The prefill configurations ([PAPER] Sec. 4.3, Table 2 shapes): M = 2048,
K = 4096, N = 14336 (the gate/up projection of a 2048-token prefill); the
vocabulary projection K = 4096, N = 128256 at M = 512; the vision-encoder
MLP up (K = 1280, N = 5120) and down (K = 5120, N = 1280) projections at
M = 1601 tokens.  Weights are the oracle-packed matrices of the parity inputs
(tests/golden/centroids.json tables, the oracle's frozen-centroid encoder),
activations the seeded N(0, 1) draws.

Each configuration runs through the three prefill paths (the fused GEMM of
s3d8_linear, the decode-then-INT8-GEMM of s3d8_linear_unfused, and the
split-K fused GEMM of s3d8_linear_splitk with the library's split count, as
the benchmark runs it) in three modes: with the INT32 accumulators requested, and without them (the kernel
builds the benchmark times, which never store accumulators) with fp32 and
with bf16 output.  Every output is compared: accumulators bit-exact, fp32
outputs bit-identical to the oracle's epilogue (the 1e-6 relative bar is
checked as well), bf16 outputs equal to the oracle's round-to-nearest-even of
its fp32 outputs.

The same three modes run on ragged shapes (row, triple and K tails, both
row-tile heights; split-K into 3 ranges) and through s3d8_forward, whose
small-M kernels are also built separately for the accumulator-free case.
Split-K is also run at the full prefill sizes with explicit split counts,
over a sweep of split counts on a ragged shape (ranges of unequal length,
one block per range, more ranges than blocks), and with one workspace
reused across calls (its counters must return to zero).
"""
import functools

import numpy as np
import pytest

import oracle
import workloads
from parity_inputs import packed_matrix, random_format

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
s3d8 = pytest.importorskip("w2_a8_matmul_amd")

REL = 1e-6


def dev(a, device):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def check_y(y_gpu, y_ref):
    y_gpu = np.asarray(y_gpu, np.float32)
    y_ref = np.asarray(y_ref, np.float32)
    err = np.abs(y_gpu.astype(np.float64) - y_ref.astype(np.float64))
    assert (err <= REL * np.abs(y_ref.astype(np.float64))).all(), float(err.max())
    assert (y_gpu[y_ref == 0] == 0).all()
    np.testing.assert_array_equal(y_gpu, y_ref)


def bf16_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


PREFILL = {"c3": workloads.C3, "lm_head_m512": workloads.C4[1], "vision_up": workloads.C4[2],
           "vision_down": workloads.C4[3]}


@functools.lru_cache(maxsize=1)
def _oracle_full(name):
    """(x, C, alpha, packed, xq, xs, acc, y) of a prefill configuration, all
    from the oracle (one configuration cached at a time: lm_head at M = 512
    holds 0.5 GB of reference outputs)."""
    lin = PREFILL[name]
    C, alpha, packed = packed_matrix(lin)
    x = workloads.activations(lin)
    xq, xs, acc, y = oracle.linear(x, packed, C, alpha, lin.N)
    return x, C, alpha, packed, xq, xs, acc, y


def _run_prefill(gpu, path, mode, x, C, alpha, packed, N):
    """One call of s3d8_linear / s3d8_linear_unfused / s3d8_linear_splitk
    ("splitk": the library's split count, "splitk<S>": S ranges); returns
    (xq, xs, acc or None, y as numpy: fp32, or bf16 bit patterns)."""
    xq, xs = s3d8.quant_act(dev(x, gpu))
    tiled = s3d8.tile(dev(packed, gpu), N)
    if path.startswith("splitk"):
        splits = int(path[6:] or 0)

        def fn(*a, **k):
            return s3d8.linear_splitk(*a, splits=splits, **k)
    else:
        fn = s3d8.linear if path == "fused" else s3d8.linear_unfused
    out = "bf16" if mode == "y_bf16" else "f32"
    if mode == "acc":
        y, acc = fn(xq, xs, tiled, dev(C, gpu), dev(alpha.view(np.int16), gpu), N, return_acc=True)
    else:
        y, acc = fn(xq, xs, tiled, dev(C, gpu), dev(alpha.view(np.int16), gpu), N, out=out), None
    torch.cuda.synchronize()
    ynp = bf16_bits(y) if out == "bf16" else y.cpu().numpy()
    return xq.cpu().numpy(), xs.cpu().numpy(), None if acc is None else acc.cpu().numpy(), ynp


def _compare(got, ref_xq, ref_xs, ref_acc, ref_y, mode):
    xq, xs, acc, y = got
    np.testing.assert_array_equal(xq, ref_xq)
    np.testing.assert_array_equal(xs, ref_xs)
    if mode == "acc":
        np.testing.assert_array_equal(acc, ref_acc)
    if mode == "y_bf16":
        np.testing.assert_array_equal(y, oracle.to_bf16(ref_y))
    else:
        check_y(y, ref_y)


@pytest.mark.parametrize("mode", ["acc", "y_f32", "y_bf16"])
@pytest.mark.parametrize("path", ["fused", "unfused", "splitk"])
@pytest.mark.parametrize("name", list(PREFILL))
def test_prefill_full_output_matches_oracle(gpu, name, path, mode):
    lin = PREFILL[name]
    x, C, alpha, packed, xq_r, xs_r, acc_r, y_r = _oracle_full(name)
    got = _run_prefill(gpu, path, mode, x, C, alpha, packed, lin.N)
    assert got[3].shape == (lin.M, lin.N)
    _compare(got, xq_r, xs_r, acc_r, y_r, mode)


# ------------------------------------------------------------------ ragged shapes, every mode
# (M, K, N): row tails of every row-tile height (1270 and 2000 take
# 160-row tiles, 600 and 640 take 128-row tiles, 300, 33 and 17 take 64-row
# tiles), ragged triples (N mod 3 = 1, 2, on every tile height), K past the
# last 64-column block, and small M through the GEMV kernels.
RAGGED = [(1270, 80, 12280), (2000, 1024, 14335), (2000, 144, 14339), (600, 80, 12280), (640, 144, 12281),
          (300, 1040, 772), (33, 1040, 97), (17, 80, 50), (16, 1040, 97), (9, 256, 48), (5, 64, 47),
          (1, 4096, 300)]


@pytest.mark.parametrize("name,splits", [("vision_down", 2), ("vision_down", 3), ("vision_down", 5),
                                         ("vision_up", 2), ("vision_up", 4), ("c3", 2)])
def test_splitk_full_output_matches_oracle(gpu, name, splits):
    """Split-K at the full prefill sizes with explicit split counts (vision
    down on 64-row tiles: 80 blocks in 2, 3 or 5 ranges; vision up on 128-row
    tiles: 20 blocks; c3 on 160-row tiles), accumulators and fp32 outputs in
    full."""
    lin = PREFILL[name]
    x, C, alpha, packed, xq_r, xs_r, acc_r, y_r = _oracle_full(name)
    got = _run_prefill(gpu, "splitk%d" % splits, "acc", x, C, alpha, packed, lin.N)
    _compare(got, xq_r, xs_r, acc_r, y_r, "acc")


@pytest.mark.parametrize("mode", ["acc", "y_f32", "y_bf16"])
@pytest.mark.parametrize("path", ["fused", "unfused", "splitk3"])
@pytest.mark.parametrize("M,K,N", RAGGED)
def test_linear_modes_ragged(gpu, M, K, N, path, mode):
    C, alpha, packed = random_format([4000, M, K, N], N, K)
    x = workloads.gaussian_matrix([4001, M, K], M, K)
    if M >= 3:
        x[2] = 0.0  # a zero token row
    xq_r, xs_r, acc_r, y_r = oracle.linear(x, packed, C, alpha, N)
    got = _run_prefill(gpu, path, mode, x, C, alpha, packed, N)
    _compare(got, xq_r, xs_r, acc_r, y_r, mode)


FWD = [(1, 4096, 14336), (2, 1040, 97), (3, 4096, 50), (4, 14336, 64), (4, 5120, 101), (8, 1280, 98),
       (16, 256, 385), (40, 256, 385)]


@pytest.mark.parametrize("mode", ["acc", "y_f32", "y_bf16"])
@pytest.mark.parametrize("M,K,N", FWD)
def test_forward_modes(gpu, M, K, N, mode):
    """s3d8_forward with and without accumulators, fp32 and bf16 output."""
    C, alpha, packed = random_format([4010, M, K, N], N, K)
    x = workloads.gaussian_matrix([4011, M, K], M, K)
    xq_r, xs_r, acc_r, y_r = oracle.linear(x, packed, C, alpha, N)
    tiled = s3d8.tile(dev(packed, gpu), N)
    out = "bf16" if mode == "y_bf16" else "f32"
    xq = torch.empty((M, K), dtype=torch.int8, device=gpu)
    xs = torch.empty((M,), dtype=torch.float32, device=gpu)
    args = (dev(x, gpu), tiled, dev(C, gpu), dev(alpha.view(np.int16), gpu), N)
    if mode == "acc":
        y, _, _, acc = s3d8.forward(*args, xq=xq, xs=xs, return_all=True, out=out)
    else:
        y = s3d8.forward(*args, xq=xq, xs=xs, out=out)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(xq.cpu().numpy(), xq_r)
    np.testing.assert_array_equal(xs.cpu().numpy(), xs_r)
    if mode == "acc":
        np.testing.assert_array_equal(acc.cpu().numpy(), acc_r)
    if out == "bf16":
        np.testing.assert_array_equal(bf16_bits(y), oracle.to_bf16(y_r))
    else:
        check_y(y.cpu().numpy(), y_r)


# K = 1040: 17 column blocks, the last one ragged (16 columns)
@pytest.mark.parametrize("splits", [2, 3, 4, 5, 7, 16, 17, 40])
@pytest.mark.parametrize("M,N", [(300, 772), (600, 12280), (33, 12280)])
def test_splitk_split_counts(gpu, M, N, splits):
    """Every split count on a ragged K: unequal ranges, one block per range
    (17), more ranges requested than blocks (40 is clamped to 17), on 64-row
    (300 x 772, 33 x 12280) and 128-row tiles (600 x 12280)."""
    K = 1040
    C, alpha, packed = random_format([4020, M, K, N], N, K)
    x = workloads.gaussian_matrix([4021, M, K], M, K)
    xq_r, xs_r, acc_r, y_r = oracle.linear(x, packed, C, alpha, N)
    got = _run_prefill(gpu, "splitk%d" % splits, "acc", x, C, alpha, packed, N)
    _compare(got, xq_r, xs_r, acc_r, y_r, "acc")


def test_splitk_workspace_reuse(gpu):
    """One zero-filled workspace across calls of different shapes and split
    counts: every result matches the oracle, and the per-tile counters are
    back at zero after each call."""
    ws = torch.zeros((s3d8.splitk_workspace_bytes(300, 5120, 1280, 5),), dtype=torch.uint8, device=gpu)
    for i, (M, K, N, splits) in enumerate([(300, 5120, 1280, 5), (300, 5120, 1280, 5), (200, 1040, 772, 3),
                                           (300, 5120, 1280, 4), (40, 640, 97, 2)]):
        C, alpha, packed = random_format([4030, i], N, K)
        x = workloads.gaussian_matrix([4031, i], M, K)
        xq_r, xs_r, acc_r, y_r = oracle.linear(x, packed, C, alpha, N)
        xq, xs = s3d8.quant_act(dev(x, gpu))
        tiled = s3d8.tile(dev(packed, gpu), N)
        y, acc = s3d8.linear_splitk(xq, xs, tiled, dev(C, gpu), dev(alpha.view(np.int16), gpu), N, splits=splits,
                                    workspace=ws, return_acc=True)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(acc.cpu().numpy(), acc_r)
        check_y(y.cpu().numpy(), y_r)
        # the counters (two int32 per tile, at most 12 tiles here) and their
        # padding fill the first 256 bytes; the partial sums follow
        assert int(ws[:256].count_nonzero()) == 0


def test_splitk_small_m_takes_gemv(gpu):
    """M <= 16 through s3d8_linear_splitk is the GEMV path of s3d8_linear
    (no workspace needed), identical results."""
    M, K, N = 8, 4096, 1000
    C, alpha, packed = random_format([4040], N, K)
    x = workloads.gaussian_matrix([4041], M, K)
    xq_r, xs_r, acc_r, y_r = oracle.linear(x, packed, C, alpha, N)
    assert s3d8.splitk_workspace_bytes(M, K, N, 4) == 0
    got = _run_prefill(gpu, "splitk4", "acc", x, C, alpha, packed, N)
    _compare(got, xq_r, xs_r, acc_r, y_r, "acc")


def test_splitk_graph_replays(gpu):
    """s3d8_linear_splitk captured in a HIP graph (as the benchmark times it):
    every replay, with eager calls on the same workspace in between, gives the
    oracle's results, and the workspace counters are back at zero after each
    (the counters are reset by the kernels themselves, no memset node)."""
    M, K, N, splits = 300, 5120, 1280, 4
    C, alpha, packed = random_format([4050], N, K)
    x = workloads.gaussian_matrix([4051], M, K)
    _, _, acc_r, y_r = oracle.linear(x, packed, C, alpha, N)
    xq, xs = s3d8.quant_act(dev(x, gpu))
    tiled = s3d8.tile(dev(packed, gpu), N)
    Cd, Sd = dev(C, gpu), dev(alpha.view(np.int16), gpu)
    ws = torch.zeros((s3d8.splitk_workspace_bytes(M, K, N, splits),), dtype=torch.uint8, device=gpu)
    y = torch.empty((M, N), dtype=torch.float32, device=gpu)
    acc = torch.empty((M, N), dtype=torch.int32, device=gpu)

    def call():
        s3d8.linear_splitk(xq, xs, tiled, Cd, Sd, N, splits=splits, workspace=ws, y=y, acc=acc, return_acc=True)

    call()  # warm-up outside the capture
    torch.cuda.synchronize()
    s = torch.cuda.Stream(device=gpu)
    s.wait_stream(torch.cuda.current_stream(gpu))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call()
    torch.cuda.synchronize()
    for rep in range(4):
        y.zero_()
        acc.zero_()
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(acc.cpu().numpy(), acc_r)
        check_y(y.cpu().numpy(), y_r)
        assert int(ws[:256].count_nonzero()) == 0
        # eager work on the same workspace between replays
        call()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(acc.cpu().numpy(), acc_r)
