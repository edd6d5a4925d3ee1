"""The library's host packer (s3d8_pack / s3d8_encode) against the oracle.

The frozen-centroid encode has a unique result given the centroid table, so
it must match the oracle bit for bit.  The k-means fit is a heuristic: on
inputs of at most 65536 vectors the library's chunked reductions reduce to
plain sequential sums, so its fit must equal the oracle's exactly; on larger
inputs it is checked by invariants (integer centroids in [0,127],
non-increasing Lloyd distortion, encode consistency with the oracle, exact
planted recovery) and by independence from the thread count.
"""
import numpy as np
import pytest

import oracle
import w2_a8_matmul_amd as s3d8
import workloads
from test_oracle_pins import _planted


SHAPES = [(1, 16), (2, 32), (3, 16), (7, 48), (64, 256), (100, 64), (385, 128)]


@pytest.mark.parametrize("N,K", SHAPES)
def test_encode_matches_oracle(N, K):
    C = workloads.uniform_centroids([1000, N, K], 0, 127)
    W = workloads.gaussian_matrix([1001, N, K], N, K, 0.02)
    W[0, 0] = -0.0
    if N > 2:
        W[2, :] = 0.0  # zero channel: alpha 0
    s_lib, p_lib = s3d8.encode(W, C)
    s_or, p_or = oracle.encode(W, C)
    np.testing.assert_array_equal(s_lib, s_or)
    np.testing.assert_array_equal(p_lib, p_or)


def test_encode_c1_rows_match_oracle():
    """Full gate/up weight shape, frozen random centroids: bit-exact encode."""
    lin = workloads.C1[1]
    W = workloads.weights(lin)[:999]
    C = workloads.random_centroids(1)
    s_lib, p_lib = s3d8.encode(W, C)
    s_or, p_or = oracle.encode(W, C)
    np.testing.assert_array_equal(s_lib, s_or)
    np.testing.assert_array_equal(p_lib, p_or)


@pytest.mark.parametrize("N,K,seed,iters", [(3, 16, 1, 5), (10, 64, 2, 30), (96, 256, 7, 40),
                                            (200, 320, 11, 25)])
def test_pack_single_chunk_equals_oracle_fit(N, K, seed, iters):
    W = workloads.gaussian_matrix([1010, N, K], N, K, 0.02)
    assert oracle.num_triples(N) * K <= 65536
    C, s, p, dist, it = s3d8.pack(W, seed=seed, max_iters=iters, return_stats=True)
    Co, cent, disto, ito = oracle.fit_centroids(W, seed, iters)
    assert it == ito
    np.testing.assert_array_equal(C, Co)
    np.testing.assert_array_equal(dist, disto)
    so, po = oracle.encode(W, Co)
    np.testing.assert_array_equal(s, so)
    np.testing.assert_array_equal(p, po)


def test_pack_planted_exact_recovery():
    C_true, alpha, W = _planted(21, 40, 2048)  # 81920 vectors: two chunks
    C, s, p, dist, it = s3d8.pack(W, seed=5, max_iters=20, return_stats=True)
    assert {tuple(r) for r in C.tolist()} == {tuple(r) for r in C_true.tolist()}
    np.testing.assert_array_equal(s, alpha)
    w = oracle.decode(p, C, W.shape[0], W.shape[1]).astype(np.float32)
    np.testing.assert_array_equal(w * oracle.bf16_to_f32(s)[:, None], W)
    assert dist[-1] == 0.0


def test_pack_multichunk_invariants_and_thread_independence():
    N, K = 300, 1024  # 100 * 1024 = 102400 vectors: two chunks
    W = workloads.gaussian_matrix([1020], N, K, 0.02)
    C1, s1, p1, d1, it1 = s3d8.pack(W, seed=3, max_iters=15, num_threads=1, return_stats=True)
    C8, s8, p8, d8, it8 = s3d8.pack(W, seed=3, max_iters=15, num_threads=8, return_stats=True)
    np.testing.assert_array_equal(C1, C8)
    np.testing.assert_array_equal(p1, p8)
    np.testing.assert_array_equal(d1, d8)
    assert C1.max() <= 127
    assert (np.diff(d1) <= 1e-12 * d1[0]).all()
    so, po = oracle.encode(W, C1)
    np.testing.assert_array_equal(s1, so)
    np.testing.assert_array_equal(p1, po)
    # the fit beats the k-means++ seeding alone
    assert d1[-1] < d1[0]


def test_pack_quality_close_to_oracle_fit():
    """Different association of the sums gives a different but comparable
    fit; the rounded tables should give reconstruction errors within 2%."""
    N, K = 300, 1024
    W = workloads.gaussian_matrix([1030], N, K, 0.02)
    C, s, p = s3d8.pack(W, seed=4, max_iters=25)
    Co, _, _, _ = oracle.fit_centroids(W, 4, 25)

    def err(C):
        a, pk = oracle.encode(W, C)
        w = oracle.decode(pk, C, N, K).astype(np.float64) * oracle.bf16_to_f32(a)[:N, None]
        return float(((w - W) ** 2).mean())

    e_lib, e_or = err(C), err(Co)
    assert abs(e_lib - e_or) <= 0.02 * e_or


def test_pack_zero_iterations_and_degenerate_inputs():
    # all-zero matrix: every vector is 0, alpha 0, signs 0, table from the
    # (uniform) seeding picks of zero vectors
    W = np.zeros((4, 16), np.float32)
    C, s, p = s3d8.pack(W, seed=1, max_iters=0)
    assert (s == 0).all() and (C == 0).all() and (p == 0).all()
    # a single channel: two padded channels in the triple
    W1 = workloads.gaussian_matrix([1040], 1, 32, 0.02)
    C, s, p = s3d8.pack(W1, seed=1, max_iters=10)
    assert s.shape == (3,) and s[1] == 0 and s[2] == 0
    so, po = oracle.encode(W1, C)
    np.testing.assert_array_equal(p, po)
