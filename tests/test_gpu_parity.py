"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bar: INT8 codes, activation scales, decoded weights and INT32 accumulators
bit-exact; fp32 outputs within 1e-6 relative error of the oracle (and zero
where the oracle's output is zero).  The epilogue is two fp32 multiplies in a
fixed order, so the outputs are also expected to be bit-identical; that is
checked too.

Small shapes are compared element by element over whole outputs; so are the
full-size decode workloads here and the full-size prefill workloads in
test_gpu_full_prefill.py.
"""
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
    t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(device)


def check_y(y_gpu, y_ref):
    y_gpu = np.asarray(y_gpu, np.float32)
    y_ref = np.asarray(y_ref, np.float32)
    err = np.abs(y_gpu.astype(np.float64) - y_ref.astype(np.float64))
    assert (err <= REL * np.abs(y_ref.astype(np.float64))).all(), float(err.max())
    assert (y_gpu[y_ref == 0] == 0).all()
    np.testing.assert_array_equal(y_gpu, y_ref)


def relayout(packed, K):
    """The tiled device layout, from its definition in include/s3d8.h:
    fragment (tile i, block b) at (i*KB + b)*1024, lane L = n + 16g owns the
    16 bytes packed[16i+n][64b+16g ..], zero past the matrix."""
    T = packed.shape[0]
    tiles, KB = (T + 15) // 16, (K + 63) // 64
    P = np.zeros((tiles * 16, KB * 64), np.uint8)
    P[:T, :K] = packed
    return P.reshape(tiles, 16, KB, 4, 16).transpose(0, 2, 3, 1, 4).reshape(-1)


def run_linear(x, C, alpha, packed, N, device, unfused=False):
    xd = dev(x, device)
    xq, xs = s3d8.quant_act(xd)
    tiled = s3d8.tile(dev(packed, device), N)
    fn = s3d8.linear_unfused if unfused else s3d8.linear
    y, acc = fn(xq, xs, tiled, dev(C, device), dev(alpha.view(np.int16), device), N, return_acc=True)
    torch.cuda.synchronize()
    return xq.cpu().numpy(), xs.cpu().numpy(), acc.cpu().numpy(), y.cpu().numpy()


def run_forward(x, C, alpha, packed, N, device):
    tiled = s3d8.tile(dev(packed, device), N)
    y, xq, xs, acc = s3d8.forward(dev(x, device), tiled, dev(C, device),
                                  dev(alpha.view(np.int16), device), N, return_all=True)
    torch.cuda.synchronize()
    return xq.cpu().numpy(), xs.cpu().numpy(), acc.cpu().numpy(), y.cpu().numpy()


# ------------------------------------------------------------------ tiled layout
@pytest.mark.parametrize("N,K", [(3, 16), (48, 64), (50, 80), (385, 1040), (14336, 4096)])
def test_tile_matches_relayout(gpu, N, K):
    _, _, packed = random_format([1990, N, K], N, K)
    tiled = s3d8.tile(dev(packed, gpu), N)
    torch.cuda.synchronize()
    assert tiled.numel() == s3d8.tiled_bytes(N, K)
    np.testing.assert_array_equal(tiled.cpu().numpy(), relayout(packed, K))


# ------------------------------------------------------------------ quant_act
def _edge_rows(K):
    x = np.zeros((6, K), np.float32)
    x[0, K // 3] = -2.5
    x[1, :] = 0.7
    x[2, :8] = [127.0, 2.5, 3.5, -2.5, -3.5, 0.5, 1.5, -0.5]
    tiny = np.float32(2.0 ** -149)
    x[4, :3] = [tiny * np.float32(100), tiny * np.float32(3), -tiny * np.float32(50)]
    x[5, :] = workloads.gaussian_matrix([2000, K], 1, K)[0] * np.float32(1e-39)  # subnormal row
    return x


# K up to 65536 runs the one-read build (the row held in registers), longer
# rows (65552, 70000) the two-read build
@pytest.mark.parametrize("M,K", [(1, 16), (1, 256), (3, 48), (8, 4096), (1, 14336), (37, 1280),
                                 (1601, 5120), (2048, 4096), (6, 16384), (7, 16400), (2, 20000),
                                 (6, 65536), (1, 65552), (7, 70000)])
def test_quant_act_matches_oracle(gpu, M, K):
    x = workloads.gaussian_matrix([2001, M, K], M, K)
    if M >= 6:
        x[:6] = _edge_rows(K)
    xq, xs = s3d8.quant_act(dev(x, gpu))
    torch.cuda.synchronize()
    xq_ref, xs_ref = oracle.quant_act(x)
    np.testing.assert_array_equal(xs.cpu().numpy(), xs_ref)
    np.testing.assert_array_equal(xq.cpu().numpy(), xq_ref)


def test_quant_act_outlier_activations(gpu):
    lin = workloads.C2[6]
    x = workloads.activations(lin, M=4)
    xq, xs = s3d8.quant_act(dev(x, gpu))
    xq_ref, xs_ref = oracle.quant_act(x)
    np.testing.assert_array_equal(xs.cpu().numpy(), xs_ref)
    np.testing.assert_array_equal(xq.cpu().numpy(), xq_ref)


# ------------------------------------------------------------------ dequant
@pytest.mark.parametrize("N,K", [(3, 16), (4, 16), (5, 48), (384, 256), (100, 1040), (1281, 5120)])
def test_dequant_matches_oracle(gpu, N, K):
    C, _, packed = random_format([2010, N, K], N, K)
    w = s3d8.dequant(dev(packed, gpu), dev(C, gpu), N)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(w.cpu().numpy(), oracle.decode(packed, C, N, K))


def test_dequant_every_byte_value(gpu):
    C = workloads.uniform_centroids([2011], 0, 127)
    packed = np.tile(np.arange(256, dtype=np.uint8), 2).reshape(2, 256)
    w = s3d8.dequant(dev(packed, gpu), dev(C, gpu), 6)
    np.testing.assert_array_equal(w.cpu().numpy(), oracle.decode(packed, C, 6, 256))


def test_dequant_full_gate_up(gpu):
    lin = workloads.C1[1]
    C, _, packed = packed_matrix(lin)
    w = s3d8.dequant(dev(packed, gpu), dev(C, gpu), lin.N)
    np.testing.assert_array_equal(w.cpu().numpy(), oracle.decode(packed, C, lin.N, lin.K))


# ------------------------------------------------------------------ linear, small
def test_linear_random_format_config(gpu):
    """M=1, K=256, N=384: random centroid table, uniform bytes, lognormal bf16 scales."""
    lin = workloads.C0
    C, alpha, packed = packed_matrix(lin)
    x = workloads.activations(lin)
    xq, xs, acc, y = run_linear(x, C, alpha, packed, lin.N, gpu)
    xq_r, xs_r, acc_r, y_r = oracle.linear(x, packed, C, alpha, lin.N)
    np.testing.assert_array_equal(xq, xq_r)
    np.testing.assert_array_equal(xs, xs_r)
    np.testing.assert_array_equal(acc, acc_r)
    check_y(y, y_r)


FUZZ = [(m, k, n) for m in (1, 2, 3, 5, 8, 9, 16, 17, 33) for (k, n) in
        [(16, 1), (16, 3), (48, 4), (64, 47), (80, 50), (256, 48), (1040, 97)]]


@pytest.mark.parametrize("M,K,N", FUZZ)
def test_linear_shape_fuzz(gpu, M, K, N):
    """Ragged N (mod 3 in {0,1,2}, partial triple tiles), K not a multiple of
    the 64-column block, M spanning one and several row tiles."""
    C, alpha, packed = random_format([2020, M, K, N], N, K)
    x = workloads.gaussian_matrix([2021, M, K], M, K)
    xq, xs, acc, y = run_linear(x, C, alpha, packed, N, gpu)
    _, _, acc_r, y_r = oracle.linear(x, packed, C, alpha, N)
    np.testing.assert_array_equal(acc, acc_r)
    check_y(y, y_r)


def test_linear_extreme_accumulators(gpu):
    """Largest magnitudes: every weight +-127, every activation code +-127,
    K = 14336: |acc| = K * 127^2 fits INT32."""
    K, N = 14336, 6
    C = np.full((32, 3), 127, np.uint8)
    packed = np.zeros((2, K), np.uint8)
    packed[0, :] = 0x3E  # all positive
    packed[1, :] = 0x7F  # all negative
    alpha = oracle.f32_to_bf16(np.full(6, 1.0, np.float32))
    x = np.full((2, K), 3.0, np.float32)
    x[1] *= -1
    xq, xs, acc, y = run_linear(x, C, alpha, packed, N, gpu)
    big = K * 127 * 127
    assert acc.tolist() == [[big] * 3 + [-big] * 3, [-big] * 3 + [big] * 3]
    _, _, acc_r, y_r = oracle.linear(x, packed, C, alpha, N)
    check_y(y, y_r)


def test_linear_zero_rows_and_zero_scales(gpu):
    K, N = 128, 10
    C, alpha, packed = random_format([2030], N, K)
    alpha[4] = 0
    x = workloads.gaussian_matrix([2031], 3, K)
    x[1] = 0
    xq, xs, acc, y = run_linear(x, C, alpha, packed, N, gpu)
    _, _, acc_r, y_r = oracle.linear(x, packed, C, alpha, N)
    np.testing.assert_array_equal(acc, acc_r)
    check_y(y, y_r)
    assert (y[1] == 0).all() and (y[:, 4] == 0).all()


# ------------------------------------------------------------------ linear, full size
def _full_compare(lin, gpu, M=None):
    M = lin.M if M is None else M
    C, alpha, packed = packed_matrix(lin)
    x = workloads.activations(lin, M)
    xq, xs, acc, y = run_linear(x, C, alpha, packed, lin.N, gpu)
    xq_r, xs_r, acc_r, y_r = oracle.linear(x, packed, C, alpha, lin.N)
    np.testing.assert_array_equal(xq, xq_r)
    np.testing.assert_array_equal(acc, acc_r)
    check_y(y, y_r)


@pytest.mark.parametrize("m", [1, 4, 8])
def test_linear_gate_up_decode(gpu, m):
    _full_compare(workloads.C1[m], gpu)


@pytest.mark.parametrize("idx", range(7))
def test_linear_decoder_layer(gpu, idx):
    _full_compare(workloads.C2[idx], gpu)


def test_linear_lm_head_decode(gpu):
    _full_compare(workloads.C4[0], gpu)


def test_linear_prefill_five_row_tiles(gpu):
    """A shape whose workgroup count makes the GEMM take 160-row tiles (5 row
    tiles per wave) on a 256-CU device: 8 row blocks instead of 10, 256
    workgroups in one round instead of 320 in two.  Ragged in every
    dimension (last row block 150 rows, K = 64 + 16, a partial last triple
    tile), compared in full."""
    M, K, N = 1270, 80, 12280
    C, alpha, packed = random_format([2090, M, K, N], N, K)
    x = workloads.gaussian_matrix([2091, M, K], M, K)
    xq, xs, acc, y = run_linear(x, C, alpha, packed, N, gpu)
    _, _, acc_r, y_r = oracle.linear(x, packed, C, alpha, N)
    np.testing.assert_array_equal(acc, acc_r)
    check_y(y, y_r)


def test_linear_repeated_calls_are_identical(gpu):
    lin = workloads.C0
    C, alpha, packed = packed_matrix(lin)
    x = workloads.activations(lin)
    outs = [run_linear(x, C, alpha, packed, lin.N, gpu)[2] for _ in range(3)]
    for o in outs[1:]:
        np.testing.assert_array_equal(o, outs[0])


# ------------------------------------------------------------------ forward (quantise + linear)
FWD = [(m, k, n) for m in (1, 2, 3, 4, 5, 6, 7, 8, 16) for (k, n) in [(16, 3), (80, 50), (1040, 97), (4096, 300),
                                                            (14336, 64), (16384, 48)]]


@pytest.mark.parametrize("M,K,N", FWD)
def test_forward_matches_oracle(gpu, M, K, N):
    """s3d8_forward: one fused launch for small M (quantisation inside the
    GEMV), quant_act + linear otherwise; both must equal the oracle."""
    C, alpha, packed = random_format([2050, M, K, N], N, K)
    x = workloads.gaussian_matrix([2051, M, K], M, K)
    if M >= 2:
        x[1] = 0.0  # an all-zero token
    xq, xs, acc, y = run_forward(x, C, alpha, packed, N, gpu)
    xq_r, xs_r, acc_r, y_r = oracle.linear(x, packed, C, alpha, N)
    np.testing.assert_array_equal(xs, xs_r)
    np.testing.assert_array_equal(xq, xq_r)
    np.testing.assert_array_equal(acc, acc_r)
    check_y(y, y_r)


@pytest.mark.parametrize("idx", range(7))
def test_forward_decoder_layer(gpu, idx):
    """The decode step of one decoder layer through s3d8_forward."""
    lin = workloads.C2[idx]
    C, alpha, packed = packed_matrix(lin)
    x = workloads.activations(lin)
    xq, xs, acc, y = run_forward(x, C, alpha, packed, lin.N, gpu)
    xq_r, xs_r, acc_r, y_r = oracle.linear(x, packed, C, alpha, lin.N)
    np.testing.assert_array_equal(xq, xq_r)
    np.testing.assert_array_equal(xs, xs_r)
    np.testing.assert_array_equal(acc, acc_r)
    check_y(y, y_r)


# ------------------------------------------------------------------ encode on the device
@pytest.mark.parametrize("N,K", [(1, 16), (3, 16), (7, 48), (100, 64), (385, 1040), (1282, 4096)])
def test_encode_device_matches_oracle(gpu, N, K):
    """Scales and bytes bit-exact, with a zero channel, -0.0, tiny and large
    entries and ties (duplicate centroid rows)."""
    C = workloads.uniform_centroids([2130, N, K], 0, 127)
    C[5] = C[3]  # duplicate rows: the lower index must win
    W = workloads.gaussian_matrix([2131, N, K], N, K, 0.02)
    W[0, 0] = -0.0
    W[0, 1] = 1e-39  # subnormal
    if N > 2:
        W[2, :] = 0.0
    if N > 5:
        W[5, 3] = 40.0
    sc, pk = s3d8.encode_device(dev(W, gpu), dev(C, gpu))
    torch.cuda.synchronize()
    s_or, p_or = oracle.encode(W, C)
    np.testing.assert_array_equal(sc.cpu().numpy().view(np.uint16), s_or)
    np.testing.assert_array_equal(pk.cpu().numpy(), p_or)


def test_encode_device_c1_gate_up(gpu):
    """The full gate/up weight matrix with the table the packer fits for it:
    the device encode reproduces the packer's bytes and scales."""
    lin = workloads.C1[1]
    W = workloads.weights(lin)
    C, alpha, packed = packed_matrix(lin)
    sc, pk = s3d8.encode_device(dev(W, gpu), dev(C, gpu))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(sc.cpu().numpy().view(np.uint16), alpha)
    np.testing.assert_array_equal(pk.cpu().numpy(), packed)


# ------------------------------------------------------------------ forward_batch
def _batch_items(specs, gpu):
    """Device inputs for (x, C, alpha, packed, N) specs."""
    items = []
    for x, C, alpha, packed, N in specs:
        items.append(dict(x=dev(x, gpu), tiled=s3d8.tile(dev(packed, gpu), N), centroids=dev(C, gpu),
                          scales=dev(alpha.view(np.int16), gpu), N=N))
    return items


def _check_batch(specs, outs):
    for (x, C, alpha, packed, N), (y, xq, xs, acc) in zip(specs, outs):
        xq_r, xs_r, acc_r, y_r = oracle.linear(x, packed, C, alpha, N)
        np.testing.assert_array_equal(xq.cpu().numpy(), xq_r)
        np.testing.assert_array_equal(xs.cpu().numpy(), xs_r)
        np.testing.assert_array_equal(acc.cpu().numpy(), acc_r)
        check_y(y.cpu().numpy(), y_r)


def test_forward_batch_decoder_layer(gpu):
    """The seven matrices of one decoder-layer step (q, o, k, v, gate, up,
    down; down has K = 14336) in one launch, each against the oracle."""
    specs = []
    for lin in workloads.C2:
        C, alpha, packed = packed_matrix(lin)
        specs.append((workloads.activations(lin), C, alpha, packed, lin.N))
    outs = s3d8.forward_batch(_batch_items(specs, gpu), return_all=True)
    torch.cuda.synchronize()
    _check_batch(specs, outs)


@pytest.mark.parametrize("M", [1, 2, 3, 4])
def test_forward_batch_ragged_shapes(gpu, M):
    """Mixed K and N (partial triple tiles, K not a multiple of 64, a matrix
    smaller than one tile) in one launch."""
    shapes = [(1040, 97), (4096, 1), (80, 50), (16, 3), (256, 385), (2064, 14336)]
    specs = []
    for i, (K, N) in enumerate(shapes):
        C, alpha, packed = random_format([2100, M, i, K, N], N, K)
        specs.append((workloads.gaussian_matrix([2101, M, i], M, K), C, alpha, packed, N))
    outs = s3d8.forward_batch(_batch_items(specs, gpu), return_all=True)
    torch.cuda.synchronize()
    _check_batch(specs, outs)


def test_forward_batch_matches_single_calls(gpu):
    """Bit-identical to one s3d8_forward per item, also for items sharing x."""
    M, K = 2, 4096
    x = workloads.gaussian_matrix([2110], M, K)
    specs = []
    for i, N in enumerate([4096, 1024, 1024]):
        C, alpha, packed = random_format([2111, i], N, K)
        specs.append((x, C, alpha, packed, N))
    items = _batch_items(specs, gpu)
    items[1]["x"] = items[0]["x"]
    items[2]["x"] = items[0]["x"]
    outs = s3d8.forward_batch(items, return_all=True)
    torch.cuda.synchronize()
    for it, (y, xq, xs, acc) in zip(items, outs):
        y1, xq1, xs1, acc1 = s3d8.forward(it["x"], it["tiled"], it["centroids"], it["scales"], it["N"],
                                          return_all=True)
        torch.cuda.synchronize()
        for a, b in [(y, y1), (xq, xq1), (xs, xs1), (acc, acc1)]:
            np.testing.assert_array_equal(a.cpu().numpy(), b.cpu().numpy())


@pytest.mark.parametrize("case", ["nine_items", "mixed_rows", "too_long_k"])
def test_forward_batch_sequential_fallback(gpu, case):
    """Item lists the one-launch kernel does not take (more than 8 items,
    different M, M * ceil(K / 1024) > 16) run as separate launches."""
    if case == "nine_items":
        dims = [(1, 64 * (i + 1), 30 + i) for i in range(9)]
    elif case == "mixed_rows":
        dims = [(1, 256, 48), (3, 256, 48)]
    else:
        dims = [(2, 16384 + 1024, 40), (2, 256, 20)]
    specs = []
    for i, (M, K, N) in enumerate(dims):
        C, alpha, packed = random_format([2120, i, M, K, N], N, K)
        specs.append((workloads.gaussian_matrix([2121, i], M, K), C, alpha, packed, N))
    outs = s3d8.forward_batch(_batch_items(specs, gpu), return_all=True)
    torch.cuda.synchronize()
    _check_batch(specs, outs)


def test_forward_gate_up_m1(gpu):
    lin = workloads.C1[1]
    C, alpha, packed = packed_matrix(lin)
    x = workloads.activations(lin)
    xq, xs, acc, y = run_forward(x, C, alpha, packed, lin.N, gpu)
    xq_r, xs_r, acc_r, y_r = oracle.linear(x, packed, C, alpha, lin.N)
    np.testing.assert_array_equal(xq, xq_r)
    np.testing.assert_array_equal(acc, acc_r)
    check_y(y, y_r)


def _half_integer_rows(K):
    """Rows whose quotients x / s sit on or one ulp beside k + 1/2: the fused
    quantiser's fast path must hand these to the exact division."""
    k = (np.arange(K) % 254) - 127                     # -127 .. 126
    half = (k + 0.5).astype(np.float32)
    rows = np.zeros((4, K), np.float32)
    rows[0] = half                                      # s = 1 exactly: x / s = k + 1/2
    rows[0, 0] = 127.0
    s = np.float32(np.float32(300.0) / np.float32(127.0))
    v = (half * s).astype(np.float32)                   # x / s within an ulp of k + 1/2
    rows[1] = np.where(np.arange(K) % 3 == 0, np.nextafter(v, np.float32(np.inf)),
                       np.where(np.arange(K) % 3 == 1, np.nextafter(v, np.float32(-np.inf)), v))
    rows[1, 1] = 300.0
    tiny = np.float32(2.0 ** -149)
    rows[2, :4] = [tiny * np.float32(100), tiny * np.float32(3), -tiny * np.float32(50), tiny * np.float32(25)]
    rows[3] = workloads.gaussian_matrix([2060, K], 1, K)[0]
    return rows


@pytest.mark.parametrize("M", [1, 2, 3, 4])
@pytest.mark.parametrize("K", [1040, 4096])
def test_forward_quantiser_rounding_boundaries(gpu, M, K):
    """The fused (one-launch) path quantises with a reciprocal and falls back
    to the IEEE quotient near rounding boundaries: codes must still equal
    the oracle's rne(x / s) for every element."""
    N = 97
    C, alpha, packed = random_format([2061, M, K], N, K)
    rows = _half_integer_rows(K)
    for first in range(4):
        x = np.ascontiguousarray(np.roll(rows, -first, axis=0)[:M])
        xq, xs, acc, y = run_forward(x, C, alpha, packed, N, gpu)
        xq_r, xs_r, acc_r, y_r = oracle.linear(x, packed, C, alpha, N)
        np.testing.assert_array_equal(xs, xs_r)
        np.testing.assert_array_equal(xq, xq_r)
        np.testing.assert_array_equal(acc, acc_r)
        check_y(y, y_r)


# ------------------------------------------------------------------ unfused prefill path
@pytest.mark.parametrize("M,K,N", FUZZ)
def test_linear_unfused_shape_fuzz(gpu, M, K, N):
    """s3d8_linear_unfused (decode to an INT8 workspace, then INT8 GEMM) on
    the same ragged shapes as the fused path."""
    C, alpha, packed = random_format([2020, M, K, N], N, K)
    x = workloads.gaussian_matrix([2021, M, K], M, K)
    xq, xs, acc, y = run_linear(x, C, alpha, packed, N, gpu, unfused=True)
    _, _, acc_r, y_r = oracle.linear(x, packed, C, alpha, N)
    np.testing.assert_array_equal(acc, acc_r)
    check_y(y, y_r)


def test_linear_unfused_extremes_and_zeros(gpu):
    K, N = 14336, 6
    C = np.full((32, 3), 127, np.uint8)
    packed = np.zeros((2, K), np.uint8)
    packed[0, :] = 0x3E
    packed[1, :] = 0x7F
    alpha = oracle.f32_to_bf16(np.full(6, 1.0, np.float32))
    x = np.full((3, K), 3.0, np.float32)
    x[1] *= -1
    x[2] = 0
    xq, xs, acc, y = run_linear(x, C, alpha, packed, N, gpu, unfused=True)
    big = K * 127 * 127
    assert acc.tolist() == [[big] * 3 + [-big] * 3, [-big] * 3 + [big] * 3, [0] * 6]
    _, _, acc_r, y_r = oracle.linear(x, packed, C, alpha, N)
    check_y(y, y_r)


def test_linear_unfused_matches_fused_full(gpu):
    """Both prefill paths produce the same accumulators and outputs on the
    full M=2048, K=4096, N=14336 problem (the oracle checks samples of it)."""
    lin = workloads.C3
    C, alpha, packed = random_format([2070], lin.N, lin.K)
    x = workloads.gaussian_matrix([2071], lin.M, lin.K)
    _, _, acc_f, y_f = run_linear(x, C, alpha, packed, lin.N, gpu)
    _, _, acc_u, y_u = run_linear(x, C, alpha, packed, lin.N, gpu, unfused=True)
    np.testing.assert_array_equal(acc_u, acc_f)
    np.testing.assert_array_equal(y_u, y_f)


def test_prefill_paths_160_row_tiles_ragged(gpu):
    """M = 2000 (12.5 tiles of 160 rows) and N = 14335 (ragged triples), the
    size at which both prefill GEMMs take 5 row tiles per wave: sampled
    entries against the oracle, and the two paths against each other in
    full."""
    M, K, N = 2000, 1024, 14335
    C, alpha, packed = random_format([2080, M, K, N], N, K)
    x = workloads.gaussian_matrix([2081, M, K], M, K)
    xq_f, xs_f, acc_f, y_f = run_linear(x, C, alpha, packed, N, gpu)
    _, _, acc_u, y_u = run_linear(x, C, alpha, packed, N, gpu, unfused=True)
    np.testing.assert_array_equal(acc_u, acc_f)
    np.testing.assert_array_equal(y_u, y_f)
    xq_r, xs_r = oracle.quant_act(x)
    np.testing.assert_array_equal(xq_f, xq_r)
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([2082])))
    ms = list(g.integers(0, M, 256)) + [0, M - 1, 1919, 1920, 1999]
    ns = list(g.integers(0, N, 256)) + [N - 1, 0, 14333, N - 1, 14334]
    ref = np.array([oracle.acc_one(xq_r[m], packed, C, K, n) for m, n in zip(ms, ns)], np.int64)
    np.testing.assert_array_equal(acc_u[np.array(ms), np.array(ns)].astype(np.int64), ref)
    for i, (m, n) in enumerate(zip(ms, ns)):
        y_r = oracle.epilogue(ref[i:i + 1].astype(np.int32).reshape(1, 1), xs_r[m:m + 1], alpha[n:n + 1], 1)
        check_y(y_u[m, n:n + 1].reshape(1, 1), y_r)


def test_linear_unfused_workspace_reuse(gpu):
    """A workspace larger than needed, reused by a second, smaller call."""
    K1, N1, K2, N2 = 1040, 97, 256, 48
    ws = torch.empty((s3d8.unfused_workspace_bytes(N1, K1),), dtype=torch.int8, device=gpu)
    for (M, K, N, seed) in [(33, K1, N1, 2080), (17, K2, N2, 2081)]:
        C, alpha, packed = random_format([seed], N, K)
        x = workloads.gaussian_matrix([seed + 100], M, K)
        xq, xs = s3d8.quant_act(dev(x, gpu))
        tiled = s3d8.tile(dev(packed, gpu), N)
        y, acc = s3d8.linear_unfused(xq, xs, tiled, dev(C, gpu), dev(alpha.view(np.int16), gpu), N,
                                     workspace=ws, return_acc=True)
        torch.cuda.synchronize()
        _, _, acc_r, y_r = oracle.linear(x, packed, C, alpha, N)
        np.testing.assert_array_equal(acc.cpu().numpy(), acc_r)
        check_y(y.cpu().numpy(), y_r)


# ------------------------------------------------------------------ tiles per workgroup
# One token row with between one and two tiles of 16 triples per CU (256 CUs
# on MI355X), where some workgroups of the streaming GEMV take a second tile:
# 257, 299, 512 and 513 tiles, K from 1040 to 14336 (one to four float4 of
# activations per lane).  Every output, the codes and the scales against the
# oracle, in both formats and output types.
ONE_TILE = [(4096, 14336), (8192, 14336), (5120, 12336), (4096, 24576), (4096, 24624), (1040, 12400),
            (14336, 12336)]


@pytest.mark.parametrize("K,N", ONE_TILE)
def test_forward_tiles_per_workgroup(gpu, K, N):
    C, alpha, packed = random_format([2140, K, N], N, K)
    x = workloads.gaussian_matrix([2141, K, N], 1, K)
    xq, xs, acc, y = run_forward(x, C, alpha, packed, N, gpu)
    xq_r, xs_r, acc_r, y_r = oracle.linear(x, packed, C, alpha, N)
    np.testing.assert_array_equal(xq, xq_r)
    np.testing.assert_array_equal(xs, xs_r)
    np.testing.assert_array_equal(acc, acc_r)
    check_y(y, y_r)


@pytest.mark.parametrize("K,N", [(4096, 14336), (8192, 12336)])
def test_forward_tiles_per_workgroup_3d8_bf16(gpu, K, N):
    _, alpha, packed = random_format([2150, K, N], N, K)
    T3 = workloads.signed_table([2151, K])
    x = workloads.gaussian_matrix([2152, K], 1, K)
    tiled = s3d8.tile(dev(packed, gpu), N)
    y, xq, xs, acc = s3d8.forward(dev(x, gpu), tiled, dev(T3, gpu), dev(alpha.view(np.int16), gpu), N,
                                  return_all=True, fmt="3d8", out="bf16")
    torch.cuda.synchronize()
    xq_r, xs_r = oracle.quant_act(x)
    acc_r = oracle.linear_acc_3d8(xq_r, packed, T3, N)
    y_r = oracle.epilogue(acc_r, xs_r, alpha, N)
    np.testing.assert_array_equal(xq.cpu().numpy(), xq_r)
    np.testing.assert_array_equal(acc.cpu().numpy(), acc_r)
    np.testing.assert_array_equal(y.view(torch.int16).cpu().numpy().view(np.uint16), oracle.to_bf16(y_r))
