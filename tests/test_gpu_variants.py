"""GPU parity of the format and output variants against the CPU oracle.

3D8 weights (blog "S3D8: a 2.7-bit weight format for fast decoding": the
whole byte indexes a (256, 3) table of signed values) and bfloat16 outputs
(blog "Fused matrix-vector product": results are converted to bf16 on the way
out), through every kernel path: the streaming GEMV (M <= 4), the fused GEMV
fallback, the GEMV on pre-quantised activations (M <= 16), the fused GEMM
(all three row-tile heights, whole and split-K), the unfused decode + INT8 GEMM
and the standalone dequantisation.

Bar: codes, scales, decoded weights and INT32 accumulators bit-exact; fp32
outputs bit-identical to the oracle (within 1e-6 relative at worst); bf16
outputs equal to the oracle's round-to-nearest-even of its fp32 outputs.
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
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def check_y(y_gpu, y_ref):
    y_gpu = np.asarray(y_gpu, np.float32)
    y_ref = np.asarray(y_ref, np.float32)
    err = np.abs(y_gpu.astype(np.float64) - y_ref.astype(np.float64))
    assert (err <= REL * np.abs(y_ref.astype(np.float64))).all(), float(err.max())
    np.testing.assert_array_equal(y_gpu, y_ref)


def bf16_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def fmt_inputs(seed, N, K, fmt):
    """(table, alpha, packed): a random S3D8 table or a random 3D8 table with
    uniform bytes and lognormal bf16 scales."""
    C, alpha, packed = random_format(seed, N, K)
    if fmt == "3d8":
        return workloads.signed_table(list(seed) + [9]), alpha, packed
    return C, alpha, packed


def oracle_path(x, table, alpha, packed, N, fmt):
    """Quantise, decode by the format, INT32 products, fp32 epilogue."""
    xq, xs = oracle.quant_act(x)
    if fmt == "3d8":
        acc = oracle.linear_acc_3d8(xq, packed, table, N)
    else:
        acc = oracle.linear_acc(xq, packed, table, N)
    return xq, xs, acc, oracle.epilogue(acc, xs, alpha, N)


def run(kind, x, table, alpha, packed, N, gpu, fmt, out):
    tiled = s3d8.tile(dev(packed, gpu), N)
    t = dev(table, gpu)
    s = dev(alpha.view(np.int16), gpu)
    if kind == "forward":
        y, xq, xs, acc = s3d8.forward(dev(x, gpu), tiled, t, s, N, return_all=True, fmt=fmt, out=out)
    elif kind == "splitk":
        xq, xs = s3d8.quant_act(dev(x, gpu))
        y, acc = s3d8.linear_splitk(xq, xs, tiled, t, s, N, splits=3, return_acc=True, fmt=fmt, out=out)
    else:
        xq, xs = s3d8.quant_act(dev(x, gpu))
        fn = s3d8.linear if kind == "linear" else s3d8.linear_unfused
        y, acc = fn(xq, xs, tiled, t, s, N, return_acc=True, fmt=fmt, out=out)
    torch.cuda.synchronize()
    ynp = bf16_bits(y) if out == "bf16" else y.cpu().numpy()
    return xq.cpu().numpy(), xs.cpu().numpy(), acc.cpu().numpy(), ynp


def compare(got, ref, out):
    xq, xs, acc, y = got
    xq_r, xs_r, acc_r, y_r = ref
    np.testing.assert_array_equal(xq, xq_r)
    np.testing.assert_array_equal(xs, xs_r)
    np.testing.assert_array_equal(acc, acc_r)
    if out == "bf16":
        np.testing.assert_array_equal(y, oracle.to_bf16(y_r))
    else:
        check_y(y, y_r)


# ------------------------------------------------------------------ dequant
@pytest.mark.parametrize("N,K", [(3, 16), (5, 48), (100, 1040), (1281, 5120)])
def test_dequant_3d8_matches_oracle(gpu, N, K):
    T3, _, packed = fmt_inputs([3000, N, K], N, K, "3d8")
    w = s3d8.dequant(dev(packed, gpu), dev(T3, gpu), N, fmt="3d8")
    torch.cuda.synchronize()
    np.testing.assert_array_equal(w.cpu().numpy(), oracle.decode_3d8(packed, T3, N, K))


def test_dequant_3d8_every_byte_value(gpu):
    T3 = workloads.signed_table([3001])
    packed = np.tile(np.arange(256, dtype=np.uint8), 2).reshape(2, 256)
    w = s3d8.dequant(dev(packed, gpu), dev(T3, gpu), 6, fmt="3d8")
    np.testing.assert_array_equal(w.cpu().numpy(), oracle.decode_3d8(packed, T3, 6, 256))


# ------------------------------------------------------------------ every path, both variants
# (kind, M, K, N): forward at M <= 4 is the streaming GEMV; at N = 200000
# (over 16 tiles per CU) the fused GEMV; M = 4 with K = 5120 and M = 8 run
# quantisation then the GEMV on quantised activations (as linear at M <= 16);
# the fused GEMM on 64-row tiles (M = 40, 300), 128-row tiles (M = 600) and
# 160-row tiles (M = 1270), also split into 3 column-block ranges (split-K;
# K = 80 has 2 blocks, so 2 ranges).
PATHS = [
    ("forward", 1, 256, 384), ("forward", 2, 1040, 97), ("forward", 3, 4096, 50), ("forward", 4, 64, 47),
    ("forward", 1, 64, 200000), ("forward", 4, 5120, 101), ("forward", 8, 1280, 98), ("linear", 1, 80, 50),
    ("linear", 16, 1040, 97),
    ("linear", 40, 256, 385), ("linear", 300, 1040, 772), ("linear", 600, 80, 12280), ("linear", 1270, 80, 12280),
    ("unfused", 40, 1040, 97), ("unfused", 129, 256, 385),
    ("splitk", 40, 1040, 97), ("splitk", 300, 1040, 772), ("splitk", 600, 1040, 12280), ("splitk", 1270, 80, 12280),
]


@pytest.mark.parametrize("fmt,out", [("3d8", "f32"), ("s3d8", "bf16"), ("3d8", "bf16")])
@pytest.mark.parametrize("kind,M,K,N", PATHS)
def test_variant_matches_oracle(gpu, kind, M, K, N, fmt, out):
    table, alpha, packed = fmt_inputs([3010, M, K, N], N, K, fmt)
    x = workloads.gaussian_matrix([3011, M, K], M, K)
    got = run(kind, x, table, alpha, packed, N, gpu, fmt, out)
    compare(got, oracle_path(x, table, alpha, packed, N, fmt), out)


def test_3d8_with_multiplied_out_table_equals_s3d8(gpu):
    """A 3D8 table holding the S3D8 decode of every byte gives the S3D8
    results bit for bit (GEMV and GEMM)."""
    K, N = 1040, 97
    C, alpha, packed = random_format([3020], N, K)
    T3 = oracle.decode(np.arange(256, dtype=np.uint8).reshape(1, 256), C, 3, 256).T.copy()
    for M in (1, 40):
        x = workloads.gaussian_matrix([3021, M], M, K)
        a = run("forward", x, C, alpha, packed, N, gpu, "s3d8", "f32")
        b = run("forward", x, T3, alpha, packed, N, gpu, "3d8", "f32")
        for u, v in zip(a, b):
            np.testing.assert_array_equal(u, v)
        compare(b, oracle_path(x, C, alpha, packed, N, "s3d8"), "f32")


def test_3d8_extreme_accumulators(gpu):
    """Table entries -127 and 127, codes +-127, K = 14336: |acc| = K * 127^2."""
    K, N = 14336, 6
    T3 = np.zeros((256, 3), np.int8)
    T3[7] = 127
    T3[200] = -127
    packed = np.zeros((2, K), np.uint8)
    packed[0, :] = 7
    packed[1, :] = 200
    alpha = oracle.f32_to_bf16(np.full(6, 1.0, np.float32))
    x = np.full((2, K), 3.0, np.float32)
    x[1] *= -1
    got = run("forward", x, T3, alpha, packed, N, gpu, "3d8", "f32")
    big = K * 127 * 127
    assert got[2].tolist() == [[big] * 3 + [-big] * 3, [-big] * 3 + [big] * 3]
    compare(got, oracle_path(x, T3, alpha, packed, N, "3d8"), "f32")


def test_bf16_output_rounding_ties(gpu):
    """Outputs exactly half-way between two bf16 values (8 significant bits)
    round to the even one: weights 1, scales 1, acc = 254 + ones."""
    K, N = 64, 3
    C = np.zeros((32, 3), np.uint8)
    C[1] = [1, 1, 1]  # byte 2: q = 1, no signs -> w = (1, 1, 1)
    packed = np.full((1, K), 2, np.uint8)
    alpha = oracle.f32_to_bf16(np.array([1.0, 1.0, 1.0], np.float32))
    # x = 127 in columns 0 and 1 and a run of ones: s = 1, acc = 254 + ones
    rows = []
    for ones in (0, 2, 3, 5, 6):
        r = np.zeros(K, np.float32)
        r[:2] = 127.0
        r[2:2 + ones] = 1.0
        rows.append(r)
    x = np.stack(rows)
    for kind in ("forward", "linear"):
        got = run(kind, x, C, alpha, packed, N, gpu, "s3d8", "bf16")
        ref = oracle_path(x, C, alpha, packed, N, "s3d8")
        assert ref[2][:, 0].tolist() == [254, 256, 257, 259, 260]
        compare(got, ref, "bf16")
        # 257 lies half-way between 256 and 258 (-> 256), 259 between 258
        # and 260 (-> 260, the even significand)
        assert got[3][:, 0].tolist() == [0x437E, 0x4380, 0x4380, 0x4382, 0x4382]


# ------------------------------------------------------------------ full size
def test_c1_gate_up_3d8_bf16_m1(gpu):
    """The c1 matrix shape (K=4096, N=14336) at one token, 3D8 with bf16
    output, compared in full."""
    lin = workloads.C1[1]
    _, alpha, packed = packed_matrix(lin)
    T3 = workloads.signed_table([3030])
    x = workloads.activations(lin, M=1)
    got = run("forward", x, T3, alpha, packed, lin.N, gpu, "3d8", "bf16")
    compare(got, oracle_path(x, T3, alpha, packed, lin.N, "3d8"), "bf16")


def test_c3_prefill_3d8_bf16_sampled_rows(gpu):
    """M = 2048, K = 4096, N = 14336 through the fused GEMM, 3D8 and bf16:
    token rows are independent, so the oracle computes sampled rows alone."""
    lin = workloads.C1[1]
    M = 2048
    _, alpha, packed = packed_matrix(lin)
    T3 = workloads.signed_table([3031])
    x = workloads.gaussian_matrix([3032], M, lin.K)
    got = run("linear", x, T3, alpha, packed, lin.N, gpu, "3d8", "bf16")
    rows = np.array([0, 1, 127, 128, 159, 160, 1023, 2047])
    ref = oracle_path(x[rows], T3, alpha, packed, lin.N, "3d8")
    compare(tuple(g[rows] for g in got), ref, "bf16")


# ------------------------------------------------------------------ 3D8 without accumulators
# The GEMMs are built separately for the call that stores no INT32
# accumulators (the one the benchmark times); the format is a run-time flag
# inside each build, so these cover the 3D8 table path of the accumulator-free
# builds: 64-row tiles (M = 300), 128-row tiles (M = 600) and 160-row tiles
# (M = 1270 and 2000, with N mod 3 = 2), whole and split into column ranges.
Y_ONLY = [("linear", 300, 1040, 772), ("linear", 600, 80, 12280), ("linear", 1270, 80, 12280),
          ("linear", 2000, 1024, 14335), ("splitk", 600, 1040, 12280)]


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("kind,M,K,N", Y_ONLY)
def test_3d8_without_accumulators_matches_oracle(gpu, kind, M, K, N, out):
    table, alpha, packed = fmt_inputs([3020, M, K, N], N, K, "3d8")
    x = workloads.gaussian_matrix([3021, M, K], M, K)
    _, _, _, y_r = oracle_path(x, table, alpha, packed, N, "3d8")
    tiled = s3d8.tile(dev(packed, gpu), N)
    t = dev(table, gpu)
    s = dev(alpha.view(np.int16), gpu)
    xq, xs = s3d8.quant_act(dev(x, gpu))
    if kind == "splitk":
        y = s3d8.linear_splitk(xq, xs, tiled, t, s, N, splits=3, fmt="3d8", out=out)
    else:
        y = s3d8.linear(xq, xs, tiled, t, s, N, fmt="3d8", out=out)
    torch.cuda.synchronize()
    if out == "bf16":
        np.testing.assert_array_equal(bf16_bits(y), oracle.to_bf16(y_r))
    else:
        check_y(y.cpu().numpy(), y_r)
