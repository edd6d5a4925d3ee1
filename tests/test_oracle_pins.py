"""Pins for the CPU oracle: each test checks the oracle against something other
than itself -- a second reading of the pages, a closed form, a library routine,
exact rational arithmetic or brute force -- so that a dropped term, a wrong
bit position, a wrong sign or a transposed operand fails at least one test.

Sources: the Graphcore blog "11 billion parameters on a phone" (sections "Bit
layout", "Fusing sign selection into lookups", "Format decoding on Arm CPUs",
"Fused matrix-vector product", "Fast? How fast?") and the paper "Llama-Mobile:
Efficient 2.7-Bit Quantization of VLMs" (Sec. 3.4 Eq. 1 and the quantisation
equations, Table 1, Sec. 4.3).
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ------------------------------------------------------------------ bit layout
def _fields_from_text(b):
    """Blog "Bit layout": S0 in bit 0, Q4..0 in bits 5..1, S1 in bit 6, and
    bit 7 holds S2 EOR S0 (so S2 = bit7 EOR bit0)."""
    s0 = b & 1
    q = (b >> 1) & 0b11111
    s1 = (b >> 6) & 1
    s2 = ((b >> 7) & 1) ^ s0
    return q, s0, s1, s2


def test_byte_fields_all_256_and_bijection():
    seen = set()
    for b in range(256):
        f = oracle.byte_fields(b)
        assert f == _fields_from_text(b), b
        assert oracle.byte_from_fields(*f) == b
        seen.add(f)
    assert len(seen) == 256


def test_byte_fields_hand_worked():
    # 0x01: only bit 0 set -> S0 = 1 and bit 7 = 0 = S2 xor S0 -> S2 = 1.
    assert oracle.byte_fields(0x01) == (0, 1, 0, 1)
    # 0x81: bit 7 = 1 -> S2 = S0 xor 1 = 0.
    assert oracle.byte_fields(0x81) == (0, 1, 0, 0)
    # 0x3E: Q = 31, no signs.
    assert oracle.byte_fields(0x3E) == (31, 0, 0, 0)
    # 0x40: only S1.
    assert oracle.byte_fields(0x40) == (0, 0, 1, 0)
    # 0x80: only the sign-difference bit -> S2 = 1 while S0 = 0.
    assert oracle.byte_fields(0x80) == (0, 0, 0, 1)


# ------------------------------------------------------------------ decode
def _signed_lut_decode(b, C):
    """Second reading of the decode, from the blog's signed-value lookup
    tables: three 64-entry tables, I0 = b AND 0x3F (table in sign-minor order:
    index = Q*2 + sign), I1 = (b >> 1) AND 0x3F (sign-major: index =
    sign*32 + Q), I2 = I0 EOR (b >> 7) (sign-minor).  A set sign selects the
    negative value."""
    C = np.asarray(C, dtype=np.int64)
    t0 = [0] * 64
    t1 = [0] * 64
    t2 = [0] * 64
    for q in range(32):
        for s in range(2):
            sign = -1 if s else 1
            t0[q * 2 + s] = sign * int(C[q, 0])
            t1[s * 32 + q] = sign * int(C[q, 1])
            t2[q * 2 + s] = sign * int(C[q, 2])
    i0 = b & 0x3F
    i1 = (b >> 1) & 0x3F
    i2 = i0 ^ (b >> 7)
    return t0[i0], t1[i1], t2[i2]


def _tables():
    yield workloads.uniform_centroids([900, 1])
    yield np.full((32, 3), 127, np.uint8)
    z = workloads.uniform_centroids([900, 2], 0, 127)
    z[::3, 1] = 0
    z[5, :] = 0
    yield z
    yield np.arange(96, dtype=np.uint8).reshape(32, 3)


@pytest.mark.parametrize("table_idx", range(4))
def test_decode_all_bytes_matches_signed_lut(table_idx):
    C = list(_tables())[table_idx]
    # one channel triple, K = 256 columns holding every byte value
    packed = np.arange(256, dtype=np.uint8).reshape(1, 256)
    w = oracle.decode(packed, C, 3, 256)
    for b in range(256):
        assert tuple(int(v) for v in w[:, b]) == _signed_lut_decode(b, C), b


def test_decode_eq1_indexing_and_ragged_n():
    """Eq. 1 with 0-based indices: channel i uses row floor(i/3) of the packed
    matrix and component i mod 3; N not a multiple of 3 drops the padded
    channels."""
    C = workloads.uniform_centroids([901])
    K, N = 5, 7  # 3 triples, last one has a single real channel
    packed = workloads.uniform_bytes([902], 3, K)
    w = oracle.decode(packed, C, N, K)
    assert w.shape == (7, 5)
    for i in range(N):
        for j in range(K):
            got = _signed_lut_decode(int(packed[i // 3, j]), C)[i % 3]
            assert w[i, j] == got
            assert oracle.decode_weight(packed, C, K, i, j) == got


def test_decode_range():
    C = np.full((32, 3), 127, np.uint8)
    packed = workloads.uniform_bytes([903], 11, 64)
    w = oracle.decode(packed, C, 33, 64)
    assert w.min() == -127 and w.max() == 127  # never -128


# ------------------------------------------------------------------ size
def _format_bytes(N, K):
    T = oracle.num_triples(N)
    return T * K + 2 * (3 * T) + 96


def test_num_triples():
    for n, t in [(1, 1), (2, 1), (3, 1), (4, 2), (384, 128), (14336, 4779), (128256, 42752),
                 (5120, 1707), (1280, 427)]:
        assert oracle.num_triples(n) == t


def test_bits_per_element_closed_form():
    """Paper Sec. 3.4: about 8/3 + 16/k bits per element; exact here as
    8 ceil(n/3) k + 16 * 3 ceil(n/3) + 768 bits over n k elements."""
    for (K, N) in [(4096, 14336), (4096, 4096), (4096, 1024), (14336, 4096), (4096, 128256),
                   (1280, 5120), (5120, 1280)]:
        bpp = 8.0 * _format_bytes(N, K) / (N * K)
        approx = 8.0 / 3.0 + 16.0 / K
        # the approximation leaves out channel padding (at most 2 channels,
        # each 8/3 bits per element plus a bf16 scale) and the 96-byte table
        pad = 3 * oracle.num_triples(N) - N
        slack = (8.0 / 3.0) * pad / N + 16.0 * pad / (N * K) + 768.0 / (N * K)
        assert approx <= bpp <= approx + slack + 1e-12
        if N >= 14336:
            assert bpp - approx < 5e-4
    # exact value for the gate/up shape
    assert _format_bytes(14336, 4096) == 19_603_554


def test_dequant_bandwidth_matches_pages():
    """The pages' S3D8 dequant read bandwidth (16.5 GB/s in 133 us) and INT8
    copy (21.2 GB/s in 310 us) follow from counting the packed bytes plus the
    bf16 channel scales, and the INT8 tensor, respectively."""
    g = _golden("dequant_bandwidth.json")
    K, N = g["shape_k"], g["shape_n"]
    T = oracle.num_triples(N)
    src = T * K + 2 * (3 * T)
    assert src == 2_195_202

    def consistent(nbytes, t_us, gbps):
        # the printed time is rounded to 1 us and the bandwidth to 0.1 GB/s
        lo = nbytes / ((t_us + 0.5) * 1e-6) / 1e9 - 0.05
        hi = nbytes / ((t_us - 0.5) * 1e-6) / 1e9 + 0.05
        return lo <= gbps <= hi

    assert consistent(src, g["s3d8_time_us"], g["s3d8_read_gbps"])
    assert consistent(N * K, g["int8_copy_time_us"], g["int8_copy_read_gbps"])
    # one byte per weight, or 4 bits per weight, would not fit the S3D8 figure
    assert not consistent(N * K, g["s3d8_time_us"], g["s3d8_read_gbps"])
    assert not consistent(N * K // 2, g["s3d8_time_us"], g["s3d8_read_gbps"])


def test_model_size_table1_consistent():
    g = _golden("model_size.json")
    bpp = g["bfloat16_bpp"] * g["s3d8_mb"] / g["bfloat16_mb"]
    assert round(bpp, 2) == g["s3d8_bpp"]
    # per-layer bpp of the model's linear shapes brackets the model average
    lo = 8.0 * _format_bytes(128256, 4096) / (128256 * 4096)
    hi = 8.0 * _format_bytes(5120, 1280) / (5120 * 1280)
    assert lo < bpp < hi + 0.005


# ------------------------------------------------------------------ bf16
def test_bf16_rne_matches_torch():
    import torch

    g = np.random.Generator(np.random.PCG64(7))
    vals = np.concatenate([
        g.standard_normal(4000).astype(np.float32) * np.float32(3.0),
        g.lognormal(-5, 3, 2000).astype(np.float32),
        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 1e-40, -1e-40, 3.0e38], np.float32),
    ])
    # exact ties: lower half exactly 0x8000 with even and odd upper halves
    ties = np.array([0x3F808000, 0x3F818000, 0x40008000, 0xBF808000], np.uint32).view(np.float32)
    vals = np.concatenate([vals, ties])
    ours = oracle.f32_to_bf16(vals)
    ref = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    back = oracle.bf16_to_f32(ours)
    np.testing.assert_array_equal(back, torch.from_numpy(vals).to(torch.bfloat16).float().numpy())


# ------------------------------------------------------------------ activations
def test_quant_act_closed_forms():
    x = np.zeros((6, 8), np.float32)
    x[0, 3] = -2.5  # one-hot
    x[1, :] = 0.7  # constant row
    # scale exactly 1.0: quotients are exact, halves round to even
    x[2, :] = [127.0, 2.5, 3.5, -2.5, -3.5, 0.5, 1.5, -0.5]
    # scale exactly 2.0
    x[3, :] = [254.0, 5.0, 7.0, -1.0, 3.0, 1.0, -9.0, 0.0]
    # row 4 all zero
    # subnormal absmax: 100 * 2^-149 / 127 rounds to 2^-149, so the absmax
    # element maps to 100, not 127 (exact IEEE, no flush to zero)
    tiny = np.float32(2.0 ** -149)
    x[5, :] = [tiny * np.float32(100), tiny * np.float32(3), 0, 0, 0, 0, 0, -tiny * np.float32(50)]
    xq, xs = oracle.quant_act(x)
    assert xq[0].tolist() == [0, 0, 0, -127, 0, 0, 0, 0]
    assert xs[0] == np.float32(2.5) / np.float32(127)
    assert xq[1].tolist() == [127] * 8
    assert xs[2] == 1.0 and xq[2].tolist() == [127, 2, 4, -2, -4, 0, 2, 0]
    assert xs[3] == 2.0 and xq[3].tolist() == [127, 2, 4, 0, 2, 0, -4, 0]
    assert xs[4] == 0.0 and not xq[4].any()
    assert xs[5] == tiny and xq[5].tolist() == [100, 3, 0, 0, 0, 0, 0, -50]


def test_quant_act_bounds_on_random_rows():
    x = workloads.activations(workloads.C2[0], M=4)
    xq, xs = oracle.quant_act(x)
    a = np.abs(x).max(axis=1)
    assert np.all(np.abs(xq.astype(np.int32)) <= 127)
    for m in range(4):
        # the absmax element maps to +-127 and the scale is within 1 ulp of a/127
        j = int(np.abs(x[m]).argmax())
        assert abs(int(xq[m, j])) == 127
        assert abs(float(xs[m]) - float(a[m]) / 127.0) <= 2.0 ** -23 * float(a[m]) / 127.0
        # each code is within half a step of the exact quotient
        err = np.abs(xq[m].astype(np.float64) - x[m].astype(np.float64) / float(xs[m]))
        assert err.max() <= 0.5 + 1e-5


# ------------------------------------------------------------------ int products
def test_linear_acc_matches_numpy_matmul():
    C = workloads.uniform_centroids([910])
    for (M, K, N) in [(1, 64, 9), (3, 48, 10), (5, 128, 31)]:
        packed = workloads.uniform_bytes([911, M, K, N], oracle.num_triples(N), K)
        x = workloads.gaussian_matrix([912, M, K, N], M, K)
        xq, _ = oracle.quant_act(x)
        w = oracle.decode(packed, C, N, K).astype(np.int64)
        ref = xq.astype(np.int64) @ w.T
        acc = oracle.linear_acc(xq, packed, C, N)
        np.testing.assert_array_equal(acc.astype(np.int64), ref)
        for (m, n) in [(0, 0), (M - 1, N - 1), (M // 2, N // 2)]:
            assert oracle.acc_one(xq[m], packed, C, K, n) == ref[m, n]


def test_linear_acc_unit_table_is_signed_sum():
    """With every centroid component equal to 1 the weights are the signs, so
    each output is a signed sum of the activation codes."""
    C = np.ones((32, 3), np.uint8)
    K, N = 96, 6
    packed = workloads.uniform_bytes([913], 2, K)
    xq = workloads.uniform_bytes([914], 2, K).astype(np.int16) - 128
    xq = np.clip(xq, -127, 127).astype(np.int8)
    acc = oracle.linear_acc(xq, packed, C, N)
    for m in range(2):
        for n in range(N):
            total = 0
            for j in range(K):
                s = _signed_lut_decode(int(packed[n // 3, j]), C)[n % 3]
                total += s * int(xq[m, j])
            assert acc[m, n] == total


def test_linear_acc_single_activation_picks_column():
    C = workloads.uniform_centroids([915])
    K, N = 32, 12
    packed = workloads.uniform_bytes([916], 4, K)
    xq = np.zeros((1, K), np.int8)
    xq[0, 17] = -3
    acc = oracle.linear_acc(xq, packed, C, N)
    for n in range(N):
        assert acc[0, n] == -3 * _signed_lut_decode(int(packed[n // 3, 17]), C)[n % 3]


def test_linear_acc_no_signs_nonnegative():
    C = workloads.uniform_centroids([917])
    K, N = 64, 9
    # bytes with bit0 = bit6 = bit7 = 0: every sign selector is 0
    packed = (workloads.uniform_bytes([918], 3, K) & 0x3E).astype(np.uint8)
    xq = np.abs(workloads.uniform_bytes([919], 1, K).astype(np.int16) - 128).clip(0, 127).astype(np.int8)
    acc = oracle.linear_acc(xq, packed, C, N)
    assert (acc >= 0).all()


def test_linear_acc_extremes_fit_int32():
    C = np.full((32, 3), 127, np.uint8)
    K, N = 14336, 3
    packed = np.full((1, K), 0x3E, np.uint8)  # all positive 127
    xq = np.full((1, K), 127, np.int8)
    acc = oracle.linear_acc(xq, packed, C, N)
    assert acc[0].tolist() == [K * 127 * 127] * 3
    packed2 = np.full((1, K), 0x7F, np.uint8)  # S0 = 1, S1 = 1, S2 = 1 -> all negative
    acc2 = oracle.linear_acc(xq, packed2, C, N)
    assert acc2[0].tolist() == [-K * 127 * 127] * 3


# ------------------------------------------------------------------ epilogue
def test_epilogue_against_fp64_and_exact_cases():
    g = np.random.Generator(np.random.PCG64(11))
    M, N = 4, 50
    acc = g.integers(-231_225_344, 231_225_344, size=(M, N)).astype(np.int32)
    acc[0, 0] = 0
    xs = (g.random(M) * 0.05).astype(np.float32)
    alpha = workloads.random_scales_bf16(77, N)
    alpha[3] = 0
    y = oracle.epilogue(acc, xs, alpha, N)
    af = oracle.bf16_to_f32(alpha).astype(np.float64)
    ref = xs.astype(np.float64)[:, None] * acc.astype(np.float64) * af[None, :]
    err = np.abs(y.astype(np.float64) - ref)
    assert (err <= 3 * 2.0 ** -24 * np.abs(ref) + 1e-45).all()
    assert y[0, 0] == 0 and (y[:, 3] == 0).all()
    # exactly representable case: 0.5 * 12 * 0.25 = 1.5
    y1 = oracle.epilogue(np.array([[12]], np.int32), np.array([0.5], np.float32),
                         oracle.f32_to_bf16(np.array([0.25], np.float32)), 1)
    assert y1[0, 0] == 1.5
    # int -> float rounds to nearest even: 2^24 + 1 -> 2^24
    y2 = oracle.epilogue(np.array([[2 ** 24 + 1]], np.int32), np.array([1.0], np.float32),
                         oracle.f32_to_bf16(np.array([1.0], np.float32)), 1)
    assert y2[0, 0] == 2.0 ** 24


def test_epilogue_order_is_left_to_right():
    """x_s * float(acc) first, then times the channel scale.  Every product of
    two fp32/bf16 values is exact in fp64, so one cast to fp32 rounds it
    correctly; search for inputs where the two associations differ."""
    g = np.random.Generator(np.random.PCG64(12))
    found = 0
    for _ in range(2000):
        acc = np.array([[int(g.integers(-2 ** 27, 2 ** 27))]], np.int32)
        xs = np.array([g.random() * 0.01], np.float32)
        ab = oracle.f32_to_bf16(np.array([g.lognormal(-5, 0.3)], np.float32))
        a = float(oracle.bf16_to_f32(ab)[0])
        facc = float(np.float32(acc[0, 0]))
        left = np.float32(float(np.float32(float(xs[0]) * facc)) * a)
        right = np.float32(float(xs[0]) * float(np.float32(facc * a)))
        if left == right:
            continue
        found += 1
        y = oracle.epilogue(acc, xs, ab, 1)
        assert y[0, 0] == left
        if found >= 20:
            break
    assert found >= 20


# ------------------------------------------------------------------ encode
def _bf16_value(h):
    return Fraction(float(oracle.bf16_to_f32(np.array([h], np.uint16))[0]))


def test_encode_brute_force_exact_rationals():
    """Frozen-centroid quantiser against brute force in exact rational
    arithmetic: alpha from the fp32 absmax/127 rounded to bf16, W' = |W|/alpha,
    q = argmin of the exact squared distance (lowest index on ties), sign
    selector = [W < 0], padded channels zero."""
    C = workloads.uniform_centroids([920], 0, 127)
    for (N, K) in [(5, 7), (6, 4), (1, 9), (8, 3)]:
        W = workloads.gaussian_matrix([921, N, K], N, K, 0.02)
        W[0, 0] = -0.0
        alpha, packed = oracle.encode(W, C)
        T = oracle.num_triples(N)
        assert alpha.shape == (3 * T,) and packed.shape == (T, K)
        amax = np.abs(W).max(axis=1)
        ref_alpha = oracle.f32_to_bf16(amax / np.float32(127.0))
        np.testing.assert_array_equal(alpha[:N], ref_alpha)
        assert (alpha[N:] == 0).all()
        for t in range(T):
            for j in range(K):
                v = []
                s = []
                for d in range(3):
                    i = 3 * t + d
                    if i < N and _bf16_value(alpha[i]) != 0:
                        v.append(Fraction(abs(float(W[i, j]))) / _bf16_value(alpha[i]))
                    else:
                        v.append(Fraction(0))
                    s.append(1 if (i < N and W[i, j] < 0) else 0)
                dists = [sum((Fraction(int(C[l, d])) - v[d]) ** 2 for d in range(3)) for l in range(32)]
                q = min(range(32), key=lambda l: (dists[l], l))
                byte = s[0] | (q << 1) | (s[1] << 6) | ((s[2] ^ s[0]) << 7)
                assert packed[t, j] == byte, (N, K, t, j)


def _planted(seed, T, K):
    """W = alpha * s * C_true[q][d] with 32 distinct integer rows, each column of
    C_true containing 127, every channel containing a 127 entry, bf16-exact
    alpha, and all 32 rows used."""
    g = np.random.Generator(np.random.PCG64(seed))
    rows = set()
    while len(rows) < 29:
        rows.add(tuple(int(v) for v in g.integers(0, 127, size=3)))
    rows = [(127, 5, 9), (3, 127, 40), (60, 2, 127)] + sorted(rows)
    C_true = np.array(rows, np.uint8)
    assert len({tuple(r) for r in C_true.tolist()}) == 32
    perm = g.permutation(32)
    C_true = C_true[perm]
    r0 = int(np.where(C_true[:, 0] == 127)[0][0])
    r1 = int(np.where(C_true[:, 1] == 127)[0][0])
    r2 = int(np.where(C_true[:, 2] == 127)[0][0])
    q = g.integers(0, 32, size=(T, K))
    q[:, 0], q[:, 1], q[:, 2] = r0, r1, r2
    q[0, 3:35] = np.arange(32)
    sgn = np.where(g.random((3 * T, K)) < 0.5, -1.0, 1.0).astype(np.float32)
    alpha = oracle.f32_to_bf16(g.lognormal(-5, 0.5, size=3 * T).astype(np.float32))
    af = oracle.bf16_to_f32(alpha)
    W = np.empty((3 * T, K), np.float32)
    for i in range(3 * T):
        W[i] = af[i] * sgn[i] * C_true[q[i // 3], i % 3].astype(np.float32)
    return C_true, alpha, W


def test_fit_planted_centroids_exact_recovery():
    T, K = 6, 40
    C_true, alpha, W = _planted(5, T, K)
    C, cent, dist, it = oracle.fit_centroids(W, seed=3, max_iters=20)
    assert {tuple(r) for r in C.tolist()} == {tuple(r) for r in C_true.tolist()}
    assert dist[-1] == 0.0
    a2, packed = oracle.encode(W, C)
    np.testing.assert_array_equal(a2, alpha)
    w = oracle.decode(packed, C, 3 * T, K).astype(np.float32)
    recon = w * oracle.bf16_to_f32(a2)[:, None]
    np.testing.assert_array_equal(recon, W)


def test_fit_invariants_gaussian():
    W = workloads.gaussian_matrix([930], 31, 200, 0.02)
    C, cent, dist, it = oracle.fit_centroids(W, seed=9, max_iters=30)
    assert C.dtype == np.uint8 and C.max() <= 127
    assert it >= 1 and len(dist) == it + 1
    d = np.asarray(dist)
    assert (np.diff(d) <= 1e-12 * d[0]).all(), d
    # the rounded table is the half-to-even rounding of the real centres, clamped
    np.testing.assert_array_equal(C, np.clip(np.round(cent), 0, 127).astype(np.uint8))
    # all normalised vectors lie in [0, 127*(1+2^-8)]^3, so the centres do too
    assert cent.min() >= 0 and cent.max() <= 127 * (1 + 2 ** -8)


def test_splitmix64_matches_published_outputs():
    """The k-means++ draws: SplitMix64 seeded with 0 gives the published first
    three outputs (the generator's own definition, not the oracle)."""
    g = _golden("splitmix64.json")
    assert [format(oracle.splitmix64(g["seed"], c), "016x") for c in (1, 2, 3)] == g["outputs_hex"]


def _u(seed, c):
    """Uniform draw c in [0, 1): the top 53 bits of SplitMix64 draw c (the
    generator is pinned against its published outputs above)."""
    return Fraction(oracle.splitmix64(seed, c) >> 11, 1 << 53)


def _points_matrix(cols):
    """W [3][K] whose triple-0 vectors are the given integer 3-vectors (one per
    input column).  Every channel holds a 127, so alpha = bf16(127/127) = 1
    exactly and the normalised vectors W' are the integers themselves."""
    W = np.array(cols, np.float32).T.copy()
    assert (W.max(axis=1) == 127).all()
    return W


def _seeded(cols, seed):
    """The 32 k-means++ centres (no Lloyd iteration), as integer tuples."""
    W = _points_matrix(cols)
    _, cent, dist, it = oracle.fit_centroids(W, seed=seed, max_iters=0)
    assert it == 0
    assert (cent == np.round(cent)).all()
    return [tuple(int(v) for v in r) for r in cent], dist


@pytest.mark.parametrize("seed", range(8))
def test_kmeanspp_first_pick_is_floor_u1_times_p(seed):
    """[PAPER] Sec. 3.4 "Quantization": k-means++ draws the first centre
    uniformly.  With P = 48 distinct vectors, centre 0 is vector
    floor(u1 * P), u1 = draw 1 (hand rule: the counter-form draw numbering
    of the fit, pick l uses draw l + 1)."""
    g = np.random.Generator(np.random.PCG64(970))
    cols = set()
    while len(cols) < 47:
        cols.add(tuple(int(v) for v in g.integers(0, 127, size=3)))
    cols = [(127, 127, 127)] + sorted(cols)
    cols = [cols[i] for i in g.permutation(48)]
    cent, _ = _seeded(cols, seed)
    first = math.floor(_u(seed, 1) * 48)
    assert cent[0] == cols[first]
    # every centre is one of the vectors, and the 32 picks are distinct
    # (48 distinct vectors: a vector already chosen has D^2 = 0)
    assert all(c in cols for c in cent) and len(set(cent)) == 32


# seeds chosen so that every branch below is taken at least twice
D2_SEEDS = [7, 14, 3, 4, 19, 25, 1, 2, 0, 13, 22, 31]


@pytest.mark.parametrize("seed", D2_SEEDS)
def test_kmeanspp_d2_pick_hand_worked(seed):
    """D^2 weighting on four vectors, worked by hand.  a = (127,127,127) twice,
    b = (127,126,127) and c = (127,127,124): |a-b|^2 = 1, |a-c|^2 = 9,
    |b-c|^2 = 10.  The first centre is vector floor(4 u1).  Each later pick
    takes the first vector whose running sum of squared distances to the
    nearest centre exceeds u * total, so with weights (w0, w1, w2, w3):
      first a: (0, 0, 1, 9), total 10: b if u2 < 1/10, else c;
      first b: (1, 1, 0, 10), total 12: a if u2 < 2/12, else c;
      first c: (9, 9, 10, 0), total 28: a if u2 < 18/28, else b.
    The third pick is the vector not yet chosen, whatever u3: it is the only
    one left with a non-zero weight.  Then every weight is 0 and pick l is
    uniform: vector floor(4 u_{l+1})."""
    a, b, c = (127, 127, 127), (127, 126, 127), (127, 127, 124)
    cols = [a, a, b, c]
    cent, dist = _seeded(cols, seed)
    u = [None] + [_u(seed, l) for l in range(1, 33)]
    first = cols[math.floor(4 * u[1])]
    if first == a:
        second = b if u[2] < Fraction(1, 10) else c
    elif first == b:
        second = a if u[2] < Fraction(2, 12) else c
    else:
        second = a if u[2] < Fraction(18, 28) else b
    third = ({a, b, c} - {first, second}).pop()
    assert cent[:3] == [first, second, third]
    for l in range(3, 32):
        assert cent[l] == cols[math.floor(4 * u[l + 1])], l
    # every vector coincides with a centre: zero distortion after seeding
    assert dist[0] == 0.0


def test_lloyd_step_hand_worked():
    """One Lloyd-Max update ([PAPER] Sec. 3.4 "Quantization": assign each
    vector to its nearest centre, move each centre to the mean of its
    vectors), worked by hand.  31 grid vectors 42 apart and a cluster of
    three near (127,127,127): n1 = (127,127,127), n2 = (127,127,125),
    n3 = (127,125,127) (34 vectors, 32 centres).  For this seed the seeding
    takes all 31 grid vectors and n1 (the cluster's other two have D^2 <= 8
    against >= 1600 for any grid vector).  The update moves n1's centre to
    the cluster mean (127, 379/3, 379/3) and leaves every grid centre (alone
    in its cell) where it is; the next assignment changes nothing, so the
    fit stops after one iteration.  Distortion: 4 + 4 = 8 after seeding,
    then 8/9 + 20/9 + 20/9 = 16/3.  The rounded table row is (127,126,126)."""
    grid = [(x, y, z) for x in (0, 42, 84, 126) for y in (0, 42, 84, 126) for z in (0, 126)]
    grid.remove((126, 126, 126))
    n1, n2, n3 = (127, 127, 127), (127, 127, 125), (127, 125, 127)
    cols = grid + [n1, n2, n3]
    seed = 4
    cent0, dist0 = _seeded(cols, seed)
    assert set(cent0) == set(grid) | {n1}
    W = _points_matrix(cols)
    C, cent, dist, it = oracle.fit_centroids(W, seed=seed, max_iters=5)
    assert it == 1
    k = cent0.index(n1)
    mean = (127.0, 379.0 / 3.0, 379.0 / 3.0)
    assert tuple(cent[k]) == mean
    for l, g0 in enumerate(cent0):
        if l != k:
            assert tuple(cent[l]) == tuple(float(v) for v in g0)
    assert dist[0] == 8.0
    assert dist[1] == pytest.approx(16.0 / 3.0, rel=1e-15)
    assert tuple(int(v) for v in C[k]) == (127, 126, 126)


def test_sign_rule_and_padding_on_encode():
    C = workloads.uniform_centroids([940], 1, 127)
    W = workloads.gaussian_matrix([941], 10, 16, 0.02)
    W[1, 2] = 0.0
    W[2, 3] = -0.0
    alpha, packed = oracle.encode(W, C)
    for i in range(12):
        for j in range(16):
            q, s0, s1, s2 = oracle.byte_fields(int(packed[i // 3, j]))
            s = (s0, s1, s2)[i % 3]
            if i >= 10:
                assert s == 0
            else:
                assert s == (1 if W[i, j] < 0 else 0)
    # decoded signs follow W wherever the decoded magnitude is nonzero
    w = oracle.decode(packed, C, 10, 16)
    nz = w != 0
    assert (np.sign(w[nz]) == np.where(W[nz] < 0, -1, 1)).all()


def test_encode_decode_idempotent():
    """A reconstructed matrix is a fixed point of the frozen-centroid quantiser
    whenever its channel scales reproduce, i.e. every channel's largest decoded
    magnitude is 127: then W' equals the chosen centroid row exactly and the
    nearest row is that row (or an identical one)."""
    C = workloads.uniform_centroids([950], 1, 126)
    C[0] = (127, 127, 127)
    W = workloads.gaussian_matrix([951], 9, 32, 0.02)
    W[:, 0] = np.where(W[:, 0] < 0, -1.0, 1.0) * 2 * np.abs(W).max(axis=1)
    alpha, packed = oracle.encode(W, C)
    w = oracle.decode(packed, C, 9, 32)
    assert (np.abs(w).max(axis=1) == 127).all()
    W2 = w.astype(np.float32) * oracle.bf16_to_f32(alpha)[:9, None]
    alpha2, packed2 = oracle.encode(W2, C)
    np.testing.assert_array_equal(alpha2, alpha)
    np.testing.assert_array_equal(oracle.decode(packed2, C, 9, 32), w)


# ------------------------------------------------------------------ 3D8 and bf16 output
# Blog "S3D8: a 2.7-bit weight format for fast decoding": 3D8 is the plain
# format with a (256, 3) table of signed values indexed by the whole byte;
# S3D8's 256 signed centroids are the 8 sign reflections of its 32
# absolute-value rows.  Blog "Fused matrix-vector product": results are
# converted to bfloat16 on the way out.
def test_3d8_with_multiplied_out_s3d8_table_reproduces_s3d8():
    """A 3D8 table whose row b is the S3D8 decode of byte b (from the
    signed-LUT reading, not from the oracle) decodes any matrix exactly as
    S3D8 does."""
    K, N = 48, 17
    packed = workloads.uniform_bytes([910], oracle.num_triples(N), K)
    for C in _tables():
        T3 = np.array([_signed_lut_decode(b, C) for b in range(256)], np.int8)
        np.testing.assert_array_equal(oracle.decode_3d8(packed, T3, N, K), oracle.decode(packed, C, N, K))


def test_3d8_decode_is_row_lookup_numpy():
    """w[3t+d][j] = T[packed[t][j]][d], checked with numpy fancy indexing; the
    table's entries differ along both axes, so reading it transposed, or
    mapping channel i to a component other than i mod 3, fails."""
    T3 = workloads.signed_table([911])
    assert (T3[:, 0] != T3[:, 1]).any() and (T3[:255] != T3[1:]).any()
    K, N = 40, 14  # ragged: 5 triples, the last with 2 real channels
    packed = workloads.uniform_bytes([912], oracle.num_triples(N), K)
    w = oracle.decode_3d8(packed, T3, N, K)
    ref = T3[packed].transpose(0, 2, 1).reshape(-1, K)[:N]
    np.testing.assert_array_equal(w, ref)
    for i, j in [(0, 0), (4, 7), (13, 39), (12, 1)]:
        assert oracle.decode_weight_3d8(packed, T3, K, i, j) == int(T3[packed[i // 3, j], i % 3])


def test_linear_acc_decoded_matches_numpy_matmul():
    g = np.random.Generator(np.random.PCG64(913))
    M, K, N = 5, 96, 13
    xq = g.integers(-127, 128, size=(M, K)).astype(np.int8)
    w = g.integers(-127, 128, size=(N, K)).astype(np.int8)
    acc = oracle.linear_acc_decoded(xq, w)
    np.testing.assert_array_equal(acc, xq.astype(np.int64) @ w.astype(np.int64).T)
    # the 3D8 product: decode by numpy indexing, multiply by numpy
    T3 = workloads.signed_table([914])
    packed = workloads.uniform_bytes([915], oracle.num_triples(N), K)
    wd = T3[packed].transpose(0, 2, 1).reshape(-1, K)[:N].astype(np.int64)
    np.testing.assert_array_equal(oracle.linear_acc_3d8(xq, packed, T3, N), xq.astype(np.int64) @ wd.T)
    # extremes: all +-127 stays within K * 127^2 and is exact
    xq_max = np.full((1, K), -127, np.int8)
    T_max = np.full((256, 3), -127, np.int8)
    assert (oracle.linear_acc_3d8(xq_max, packed, T_max, N) == K * 127 * 127).all()


def test_to_bf16_matches_torch_and_scalar():
    import torch

    g = np.random.Generator(np.random.PCG64(916))
    vals = np.concatenate([
        g.standard_normal(3000).astype(np.float32) * np.float32(40.0),
        g.lognormal(-8, 4, 991).astype(np.float32),
        np.array([0.0, -0.0, 1.0, 1e-40, -3.0e38], np.float32),
        # exact ties (lower half 0x8000) with even and odd upper halves
        np.array([0x3F808000, 0x3F818000, 0xC0008000, 0x00018000], np.uint32).view(np.float32),
    ]).reshape(40, -1)
    ours = oracle.to_bf16(vals)
    ref = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(ours.reshape(-1)[:200], oracle.f32_to_bf16(vals.reshape(-1)[:200]))
    assert list(oracle.to_bf16(np.array([0x3F808000, 0x3F818000], np.uint32).view(np.float32))) == [0x3F80, 0x3F82]
