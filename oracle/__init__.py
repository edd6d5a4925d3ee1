"""Plain CPU oracle for the S3D8 weight-decode-fused linear layer.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``.  The product library never imports,
links or runs anything here, and nothing here imports the product package.

The arithmetic lives in ``oracle.c`` (plain scalar C, fp64 where the pages do
not fix a precision, fp32 where they do).  This module only loads it with
ctypes and marshals numpy arrays.  Each function names the passage it
follows; see the header of ``oracle.c`` for the sources and readings.

Parity status of each function (what pins it, in ``tests/test_oracle_pins.py``):
  byte_fields / byte_from_fields  pinned (exhaustive 256-byte bijection and the
                                  signed-LUT index construction of the blog)
  decode / decode_weight          pinned (256 bytes x several tables against the
                                  LUT construction; planted recovery)
  quant_act                       pinned (closed forms: one-hot, constant rows,
                                  exact half-way quotients, zero/subnormal rows)
  linear_acc / acc_one            pinned (numpy int64 matmul; C == 1 signed sum;
                                  single nonzero activation)
  epilogue                        pinned (fp64 evaluation within 2 ulp, zeros)
  channel_scales / f32_to_bf16    pinned (torch bfloat16 conversion; exact
                                  planted scales)
  encode                          pinned (brute-force argmin on tiny inputs,
                                  sign rule, planted recovery)
  decode_3d8 / decode_weight_3d8  pinned (a 3D8 table holding the S3D8 decode of
                                  every byte reproduces the S3D8 decode; numpy
                                  fancy indexing of distinct-valued tables)
  linear_acc_decoded              pinned (numpy int64 matmul)
  to_bf16                         pinned (torch bfloat16 conversion; ties to
                                  even on constructed half-way values)
  fit_centroids                   invariants only: integer centroids in
                                  [0,127], non-increasing Lloyd distortion,
                                  exact planted recovery.  Fit quality on
                                  Gaussian weights: parity unpinned (the pages
                                  print no centroid values or errors).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
# ORACLE_LIB selects another build of oracle.c (e.g. the sanitizer build)
_LIB = os.environ.get("ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into oracle/liboracle.so with gcc (no GPU needed)."""
    if not force and os.path.exists(_LIB):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-ffp-contract=off", "-fno-fast-math", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build(force=True)
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    I32 = ctypes.c_int32
    U64 = ctypes.c_uint64
    sig = {
        "oracle_bf16_to_f32": (ctypes.c_float, [ctypes.c_uint16]),
        "oracle_f32_to_bf16_rne": (ctypes.c_uint16, [ctypes.c_float]),
        "oracle_byte_fields": (None, [ctypes.c_uint8, P, P, P, P]),
        "oracle_byte_from_fields": (ctypes.c_uint8, [I32, I32, I32, I32]),
        "oracle_decode_weight": (I32, [P, P, I64, I64, I64]),
        "oracle_decode": (None, [P, P, I64, I64, P]),
        "oracle_decode_weight_3d8": (I32, [P, P, I64, I64, I64]),
        "oracle_decode_3d8": (None, [P, P, I64, I64, P]),
        "oracle_linear_acc_decoded": (I32, [P, I64, I64, I64, P, P]),
        "oracle_to_bf16": (None, [P, I64, P]),
        "oracle_quant_act": (None, [P, I64, I64, P, P]),
        "oracle_acc_one": (I64, [P, P, P, I64, I64]),
        "oracle_linear_acc": (I32, [P, I64, I64, I64, P, P, P]),
        "oracle_epilogue": (None, [P, P, P, I64, I64, P]),
        "oracle_num_triples": (I64, [I64]),
        "oracle_channel_scales": (None, [P, I64, I64, P]),
        "oracle_encode": (None, [P, I64, I64, P, P, P]),
        "oracle_splitmix64": (U64, [U64, U64]),
        "oracle_fit_centroids": (I32, [P, I64, I64, P, U64, I32, P, P, P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------- scalars
def bf16_to_f32(h) -> np.ndarray:
    """bf16 bit patterns (uint16) -> fp32 values."""
    h = _c(h, np.uint16)
    lib = _load()
    out = np.empty(h.shape, np.float32)
    flat_h, flat_o = h.reshape(-1), out.reshape(-1)
    for i in range(flat_h.size):
        flat_o[i] = lib.oracle_bf16_to_f32(int(flat_h[i]))
    return out


def f32_to_bf16(f) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even."""
    f = _c(f, np.float32)
    lib = _load()
    out = np.empty(f.shape, np.uint16)
    flat_f, flat_o = f.reshape(-1), out.reshape(-1)
    for i in range(flat_f.size):
        flat_o[i] = lib.oracle_f32_to_bf16_rne(float(flat_f[i]))
    return out


def byte_fields(b: int):
    """Blog "Bit layout": byte -> (q, S0, S1, S2)."""
    lib = _load()
    vals = [ctypes.c_int32() for _ in range(4)]
    lib.oracle_byte_fields(ctypes.c_uint8(b), *[ctypes.byref(v) for v in vals])
    return tuple(v.value for v in vals)


def byte_from_fields(q: int, s0: int, s1: int, s2: int) -> int:
    return int(_load().oracle_byte_from_fields(q, s0, s1, s2))


def num_triples(n: int) -> int:
    return int(_load().oracle_num_triples(n))


# ---------------------------------------------------------------- decode
def decode_weight(packed, C, K: int, i: int, j: int) -> int:
    packed = _c(packed, np.uint8)
    C = _c(C, np.uint8)
    return int(_load().oracle_decode_weight(_p(packed), _p(C), K, i, j))


def decode(packed, C, N: int, K: int) -> np.ndarray:
    """Eq. 1 (without alpha), one weight at a time: int8 [N][K]."""
    packed = _c(packed, np.uint8)
    C = _c(C, np.uint8)
    assert packed.size == num_triples(N) * K and C.size == 96
    w = np.empty((N, K), np.int8)
    _load().oracle_decode(_p(packed), _p(C), N, K, _p(w))
    return w


def decode_weight_3d8(packed, T3, K: int, i: int, j: int) -> int:
    packed = _c(packed, np.uint8)
    T3 = _c(T3, np.int8)
    return int(_load().oracle_decode_weight_3d8(_p(packed), _p(T3), K, i, j))


def decode_3d8(packed, T3, N: int, K: int) -> np.ndarray:
    """3D8 (blog "S3D8 design notes"): w[3t+d][j] = T3[packed[t][j]][d], int8 [N][K]."""
    packed = _c(packed, np.uint8)
    T3 = _c(T3, np.int8)
    assert packed.size == num_triples(N) * K and T3.size == 768
    w = np.empty((N, K), np.int8)
    _load().oracle_decode_3d8(_p(packed), _p(T3), N, K, _p(w))
    return w


# ---------------------------------------------------------------- activations
def quant_act(x):
    """Per-token absmax INT8: returns (xq int8 [M][K], xs fp32 [M])."""
    x = _c(x, np.float32)
    M, K = x.shape
    xq = np.empty((M, K), np.int8)
    xs = np.empty((M,), np.float32)
    _load().oracle_quant_act(_p(x), M, K, _p(xq), _p(xs))
    return xq, xs


# ---------------------------------------------------------------- products
def acc_one(xq_row, packed, C, K: int, n: int) -> int:
    xq_row = _c(xq_row, np.int8)
    packed = _c(packed, np.uint8)
    C = _c(C, np.uint8)
    assert xq_row.size == K
    return int(_load().oracle_acc_one(_p(xq_row), _p(packed), _p(C), K, n))


def linear_acc(xq, packed, C, N: int) -> np.ndarray:
    """Naive int dot products of xq [M][K] with the decoded weights: int32 [M][N]."""
    xq = _c(xq, np.int8)
    packed = _c(packed, np.uint8)
    C = _c(C, np.uint8)
    M, K = xq.shape
    assert packed.size == num_triples(N) * K
    acc = np.empty((M, N), np.int32)
    bad = _load().oracle_linear_acc(_p(xq), M, K, N, _p(packed), _p(C), _p(acc))
    if bad:
        raise ArithmeticError("accumulator outside K*127^2")
    return acc


def linear_acc_decoded(xq, w) -> np.ndarray:
    """Naive int dot products of xq [M][K] with a decoded int8 matrix w [N][K]."""
    xq = _c(xq, np.int8)
    w = _c(w, np.int8)
    M, K = xq.shape
    N = w.shape[0]
    assert w.shape == (N, K)
    acc = np.empty((M, N), np.int32)
    bad = _load().oracle_linear_acc_decoded(_p(xq), M, K, N, _p(w), _p(acc))
    if bad:
        raise ArithmeticError("accumulator outside K*127^2")
    return acc


def linear_acc_3d8(xq, packed, T3, N: int) -> np.ndarray:
    """INT32 products with 3D8 weights: decode, then plain dot products."""
    xq = _c(xq, np.int8)
    return linear_acc_decoded(xq, decode_3d8(packed, T3, N, xq.shape[1]))


def to_bf16(y) -> np.ndarray:
    """bf16 output of the blog's kernel: RNE of each fp32 result (uint16 bits)."""
    y = _c(y, np.float32)
    out = np.empty(y.shape, np.uint16)
    _load().oracle_to_bf16(_p(y), y.size, _p(out))
    return out


def epilogue(acc, xs, alpha_bf16, N: int) -> np.ndarray:
    """y = xs * float(acc) * float(alpha) in fp32, for the first N channels."""
    acc = _c(acc, np.int32)
    xs = _c(xs, np.float32)
    alpha_bf16 = _c(alpha_bf16, np.uint16)
    M = acc.shape[0]
    assert acc.shape == (M, N) and alpha_bf16.size >= N and xs.size == M
    y = np.empty((M, N), np.float32)
    _load().oracle_epilogue(_p(acc), _p(xs), _p(alpha_bf16), M, N, _p(y))
    return y


def linear(x, packed, C, alpha_bf16, N: int):
    """The whole path: quantise x, INT32 products, fp32 epilogue."""
    xq, xs = quant_act(x)
    acc = linear_acc(xq, packed, C, N)
    y = epilogue(acc, xs, alpha_bf16, N)
    return xq, xs, acc, y


# ---------------------------------------------------------------- packing
def channel_scales(W) -> np.ndarray:
    W = _c(W, np.float32)
    N, K = W.shape
    alpha = np.empty((3 * num_triples(N),), np.uint16)
    _load().oracle_channel_scales(_p(W), N, K, _p(alpha))
    return alpha


def encode(W, C):
    """Frozen-centroid quantiser: returns (alpha bf16 [3*N3], packed [N3][K])."""
    W = _c(W, np.float32)
    C = _c(C, np.uint8)
    N, K = W.shape
    T = num_triples(N)
    alpha = np.empty((3 * T,), np.uint16)
    packed = np.empty((T, K), np.uint8)
    _load().oracle_encode(_p(W), N, K, _p(C), _p(alpha), _p(packed))
    return alpha, packed


def fit_centroids(W, seed: int, max_iters: int):
    """k-means++ / Lloyd-Max fit.  Returns (C uint8 [32][3], centres fp64
    [32][3], distortion fp64 [iters+1], iters)."""
    W = _c(W, np.float32)
    N, K = W.shape
    alpha = channel_scales(W)
    C = np.empty((32, 3), np.uint8)
    cent = np.empty((32, 3), np.float64)
    dist = np.zeros((max_iters + 1,), np.float64)
    it = _load().oracle_fit_centroids(_p(W), N, K, _p(alpha), seed, max_iters,
                                      _p(C), _p(cent), _p(dist))
    if it < 0:
        raise MemoryError("oracle_fit_centroids")
    return C, cent, dist[: it + 1], it


def pack(W, seed: int, max_iters: int):
    """Fit then encode: (C, alpha, packed)."""
    C, _, _, _ = fit_centroids(W, seed, max_iters)
    alpha, packed = encode(W, C)
    return C, alpha, packed


def splitmix64(seed: int, c: int) -> int:
    return int(_load().oracle_splitmix64(seed, c))
