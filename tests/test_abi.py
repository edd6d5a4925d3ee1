"""The C ABI on the host (no GPU): the library loads, exports every symbol
declared in include/s3d8.h with the expected behaviour of its size helpers,
and every device entry point rejects bad arguments before touching the GPU."""
import ctypes
import os
import re

import numpy as np
import pytest

import w2_a8_matmul_amd as s3d8
from w2_a8_matmul_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    with open(os.path.join(ROOT, "include", "s3d8.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(s3d8_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_expected_entry_points():
    syms = _declared_symbols()
    for name in ["s3d8_pack", "s3d8_encode", "s3d8_quant_act", "s3d8_linear", "s3d8_dequant",
                 "s3d8_last_error", "s3d8_num_triples", "s3d8_packed_bytes", "s3d8_format_bytes",
                 "s3d8_version"]:
        assert name in syms


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(_lib.LIB_PATH)
    for name in _declared_symbols():
        assert hasattr(lib, name), name
        assert name in _lib.SIGNATURES, name


def test_exported_symbols_are_c_linkage():
    out = os.popen(f"nm -D --defined-only {_lib.LIB_PATH}").read()
    exported = set(re.findall(r"\bT (s3d8_[a-z0-9_]+)$", out, flags=re.M))
    assert set(_declared_symbols()) <= exported


def test_size_helpers():
    L = _lib.lib()
    assert L.s3d8_version() >= 10000
    assert L.s3d8_num_triples(14336) == 4779
    assert L.s3d8_num_triples(384) == 128
    assert L.s3d8_num_triples(0) == -1
    assert L.s3d8_packed_bytes(14336, 4096) == 4779 * 4096
    assert L.s3d8_format_bytes(14336, 4096) == 19_603_554
    assert L.s3d8_format_bytes(128256, 4096) == 175_368_800
    assert L.s3d8_packed_bytes(-1, 16) == -1


def _err(name, *args):
    rc = getattr(_lib.lib(), name)(*args)
    msg = _lib.lib().s3d8_last_error().decode()
    return rc, msg


# Fake device-looking addresses: validation must fail before any dereference
# or HIP call, so these are never touched.
A16 = 0x10000
A_ODD = 0x10001


def test_quant_act_validation():
    assert _err("s3d8_quant_act", None, 1, 16, A16, A16, None)[0] == _lib.S3D8_ERR_INVALID_ARG
    assert _err("s3d8_quant_act", A16, 0, 16, A16, A16, None)[0] == _lib.S3D8_ERR_INVALID_ARG
    rc, msg = _err("s3d8_quant_act", A16, 1, 24, A16, A16, None)
    assert rc == _lib.S3D8_ERR_SHAPE and "16" in msg
    assert _err("s3d8_quant_act", A_ODD, 1, 16, A16, A16, None)[0] == _lib.S3D8_ERR_ALIGN


TB = 1 << 40  # a tiled_bytes large enough for every shape below


def test_linear_validation():
    good = dict(xq=A16, xs=A16, M=1, K=64, N=9, packed=A16, tb=TB, C=A16, s=A16, y=A16, acc=None)

    def call(**kw):
        a = dict(good, **kw)
        return _err("s3d8_linear", a["xq"], a["xs"], a["M"], a["K"], a["N"], a["packed"], a["tb"], a["C"],
                    a["s"], a["y"], a["acc"], None)[0]

    assert call(xq=None) == _lib.S3D8_ERR_INVALID_ARG
    assert call(y=None) == _lib.S3D8_ERR_INVALID_ARG
    assert call(C=None) == _lib.S3D8_ERR_INVALID_ARG
    assert call(M=0) == _lib.S3D8_ERR_INVALID_ARG
    assert call(N=-3) == _lib.S3D8_ERR_INVALID_ARG
    assert call(K=40) == _lib.S3D8_ERR_SHAPE
    assert call(packed=A_ODD) == _lib.S3D8_ERR_ALIGN
    assert call(xq=A_ODD) == _lib.S3D8_ERR_ALIGN
    assert call(C=A16 + 2) == _lib.S3D8_ERR_ALIGN
    assert call(M=1 << 31) == _lib.S3D8_ERR_SHAPE
    assert call(N=1 << 30, K=1 << 12) == _lib.S3D8_ERR_SHAPE


@pytest.mark.parametrize("entry", ["s3d8_linear", "s3d8_forward", "s3d8_linear_unfused", "s3d8_linear_ex",
                                   "s3d8_forward_ex", "s3d8_linear_unfused_ex", "s3d8_forward_batch"])
def test_canonical_buffer_rejected_as_tiled(entry):
    """A buffer of the canonical packed size ceil(N/3) * K passed where the
    tiled layout is expected is refused (INVALID_ARG) before any GPU work:
    at c1 (N = 14336, K = 4096) the canonical matrix is 19,574,784 bytes and
    the tiled one 19,595,264."""
    L = _lib.lib()
    N, K = 14336, 4096
    canon, tiled = L.s3d8_packed_bytes(N, K), L.s3d8_tiled_bytes(N, K)
    assert canon < tiled
    ws = L.s3d8_unfused_workspace_bytes(N, K)

    def call(tb):
        if entry == "s3d8_linear":
            return L.s3d8_linear(A16, A16, 1, K, N, A16, tb, A16, A16, A16, None, None)
        if entry == "s3d8_forward":
            return L.s3d8_forward(A16, 1, K, N, A16, tb, A16, A16, A16, A16, A16, None, None)
        if entry == "s3d8_linear_unfused":
            return L.s3d8_linear_unfused(A16, A16, 40, K, N, A16, tb, A16, A16, A16, None, A16, ws, None)
        if entry == "s3d8_linear_ex":
            return L.s3d8_linear_ex(A16, A16, 1, K, N, A16, tb, A16, 1, A16, A16, 1, None, None)
        if entry == "s3d8_forward_ex":
            return L.s3d8_forward_ex(A16, 1, K, N, A16, tb, A16, 1, A16, A16, 1, A16, A16, None, None)
        if entry == "s3d8_linear_unfused_ex":
            return L.s3d8_linear_unfused_ex(A16, A16, 40, K, N, A16, tb, A16, 0, A16, A16, 1, None, A16, ws, None)
        item = _lib.ForwardItem(x=A16, M=1, K=K, N=N, tiled=A16, tiled_bytes=tb, centroids=A16, scales_bf16=A16,
                                y=A16, xq=A16, xs=A16, acc_out=None)
        items = (_lib.ForwardItem * 1)(item)
        return L.s3d8_forward_batch(1, ctypes.addressof(items), None)

    assert call(canon) == _lib.S3D8_ERR_INVALID_ARG
    assert "tiled" in L.s3d8_last_error().decode()
    assert call(tiled - 1) == _lib.S3D8_ERR_INVALID_ARG
    assert call(0) == _lib.S3D8_ERR_INVALID_ARG


def test_tile_and_forward_validation():
    L = _lib.lib()
    assert L.s3d8_tiled_bytes(14336, 4096) == 299 * 64 * 1024
    assert L.s3d8_tiled_bytes(3, 16) == 1024
    assert L.s3d8_tiled_bytes(0, 16) == -1
    assert L.s3d8_tile(None, 3, 16, A16, None) == _lib.S3D8_ERR_INVALID_ARG
    assert L.s3d8_tile(A16, 3, 24, A16, None) == _lib.S3D8_ERR_SHAPE
    assert L.s3d8_tile(A16, 3, 16, A_ODD, None) == _lib.S3D8_ERR_ALIGN
    assert L.s3d8_tile(A16, 1 << 31, 4096, A16, None) == _lib.S3D8_ERR_SHAPE

    def fwd(**kw):
        a = dict(x=A16, M=1, K=64, N=9, t=A16, tb=TB, C=A16, s=A16, y=A16, xq=A16, xs=A16, acc=None)
        a.update(kw)
        return L.s3d8_forward(a["x"], a["M"], a["K"], a["N"], a["t"], a["tb"], a["C"], a["s"], a["y"], a["xq"],
                              a["xs"], a["acc"], None)

    assert fwd(x=None) == _lib.S3D8_ERR_INVALID_ARG
    assert fwd(xq=None) == _lib.S3D8_ERR_INVALID_ARG
    assert fwd(xs=None) == _lib.S3D8_ERR_INVALID_ARG
    assert fwd(K=8) == _lib.S3D8_ERR_SHAPE
    assert fwd(x=A_ODD) == _lib.S3D8_ERR_ALIGN
    assert fwd(t=A_ODD) == _lib.S3D8_ERR_ALIGN
    assert fwd(C=A16 + 1) == _lib.S3D8_ERR_ALIGN


def test_dequant_validation():
    L = _lib.lib()
    assert L.s3d8_dequant(None, A16, 3, 16, A16, None) == _lib.S3D8_ERR_INVALID_ARG
    assert L.s3d8_dequant(A16, A16, 3, 8, A16, None) == _lib.S3D8_ERR_SHAPE
    assert L.s3d8_dequant(A16, A16, 3, 16, A_ODD, None) == _lib.S3D8_ERR_ALIGN
    assert L.s3d8_dequant(A16, A16 + 1, 3, 16, A16, None) == _lib.S3D8_ERR_ALIGN
    assert L.s3d8_dequant(A16, A16, 0, 16, A16, None) == _lib.S3D8_ERR_INVALID_ARG


def test_hbm_read_probe_validation():
    L = _lib.lib()
    assert L.s3d8_hbm_read_probe(None, 16, 1, A16, None) == _lib.S3D8_ERR_INVALID_ARG
    assert L.s3d8_hbm_read_probe(A16, 16, 1, None, None) == _lib.S3D8_ERR_INVALID_ARG
    assert L.s3d8_hbm_read_probe(A16, 0, 1, A16, None) == _lib.S3D8_ERR_INVALID_ARG
    assert L.s3d8_hbm_read_probe(A16, 24, 1, A16, None) == _lib.S3D8_ERR_INVALID_ARG
    assert L.s3d8_hbm_read_probe(A16, 16, 0, A16, None) == _lib.S3D8_ERR_INVALID_ARG
    assert L.s3d8_hbm_read_probe(A16, 16, 65537, A16, None) == _lib.S3D8_ERR_INVALID_ARG
    assert L.s3d8_hbm_read_probe(A_ODD, 16, 1, A16, None) == _lib.S3D8_ERR_ALIGN
    assert L.s3d8_hbm_read_probe(A16, 16, 1, A16 + 2, None) == _lib.S3D8_ERR_ALIGN


def test_noalloc_validation():
    """s3d8_linear_unfused_noalloc refuses, before any GPU work, a matrix
    whose decoded size exceeds its 64 MiB device scratch, and validates the
    rest like s3d8_linear_unfused."""
    L = _lib.lib()
    assert _lib.S3D8_NOALLOC_SCRATCH_BYTES == 64 * 2 ** 20
    with open(os.path.join(ROOT, "include", "s3d8.h")) as f:
        assert "#define S3D8_NOALLOC_SCRATCH_BYTES (64LL * 1024 * 1024)" in f.read()
    K, N = 4096, 128256
    assert L.s3d8_unfused_workspace_bytes(N, K) > _lib.S3D8_NOALLOC_SCRATCH_BYTES
    rc = L.s3d8_linear_unfused_noalloc(A16, A16, 17, K, N, A16, TB, A16, A16, A16, None, None)
    assert rc == _lib.S3D8_ERR_SHAPE and "scratch" in L.s3d8_last_error().decode()
    assert L.s3d8_linear_unfused_noalloc(A16, A16, 1, 24, 9, A16, TB, A16, A16, A16, None, None) \
        == _lib.S3D8_ERR_SHAPE
    assert L.s3d8_linear_unfused_noalloc(A_ODD, A16, 1, 64, 9, A16, TB, A16, A16, A16, None, None) \
        == _lib.S3D8_ERR_ALIGN
    assert L.s3d8_linear_unfused_noalloc(A16, A16, 1, 4096, 14336, A16, 1000, A16, A16, A16, None, None) \
        == _lib.S3D8_ERR_INVALID_ARG
    assert L.s3d8_linear_unfused_noalloc(A16, A16, 0, 64, 9, A16, TB, A16, A16, A16, None, None) \
        == _lib.S3D8_ERR_INVALID_ARG


def test_mfma_rate_probe_validation():
    L = _lib.lib()
    assert L.s3d8_mfma_rate_probe(1, 1, 1, None, None) == _lib.S3D8_ERR_INVALID_ARG
    assert L.s3d8_mfma_rate_probe(0, 1, 1, A16, None) == _lib.S3D8_ERR_INVALID_ARG
    assert L.s3d8_mfma_rate_probe(1, 0, 1, A16, None) == _lib.S3D8_ERR_INVALID_ARG
    assert L.s3d8_mfma_rate_probe(1, 65537, 1, A16, None) == _lib.S3D8_ERR_INVALID_ARG
    assert L.s3d8_mfma_rate_probe(1, 1, 128, A16, None) == _lib.S3D8_ERR_INVALID_ARG
    assert L.s3d8_mfma_rate_probe(1, 1, -129, A16, None) == _lib.S3D8_ERR_INVALID_ARG
    assert L.s3d8_mfma_rate_probe(1, 1, 1, A16 + 2, None) == _lib.S3D8_ERR_ALIGN


def test_linear_unfused_validation():
    L = _lib.lib()
    assert L.s3d8_unfused_workspace_bytes(10, 64) == 2048  # 12 channels: one 32-channel fragment
    assert L.s3d8_unfused_workspace_bytes(14336, 4096) == 449 * 64 * 2048
    assert L.s3d8_unfused_workspace_bytes(0, 64) == -1
    need = L.s3d8_unfused_workspace_bytes(9, 64)

    def call(ws=A16, nbytes=need, xq=A16, K=64):
        return L.s3d8_linear_unfused(xq, A16, 1, K, 9, A16, TB, A16, A16, A16, None, ws, nbytes, None)

    assert call(ws=None) == _lib.S3D8_ERR_INVALID_ARG
    assert call(nbytes=need - 1) == _lib.S3D8_ERR_INVALID_ARG
    assert call(ws=A_ODD) == _lib.S3D8_ERR_ALIGN
    assert call(xq=A_ODD) == _lib.S3D8_ERR_ALIGN
    assert call(K=24) == _lib.S3D8_ERR_SHAPE
    assert call(nbytes=need - 1) == _lib.S3D8_ERR_INVALID_ARG
    assert b"workspace" in L.s3d8_last_error()
    # a decoded matrix over 2^31 bytes is refused before any device work
    assert L.s3d8_linear_unfused(A16, A16, 1, 16384, 400000, A16, TB, A16, A16, A16, None, A16, 1 << 40,
                                 None) == _lib.S3D8_ERR_SHAPE


def test_forward_batch_validation():
    L = _lib.lib()
    assert L.s3d8_forward_batch(0, None, None) == 0  # nothing to do, no device touched
    assert L.s3d8_forward_batch(-1, None, None) == _lib.S3D8_ERR_INVALID_ARG
    assert L.s3d8_forward_batch(1, None, None) == _lib.S3D8_ERR_INVALID_ARG
    good = dict(x=A16, M=1, K=64, N=9, tiled=A16, tiled_bytes=TB, centroids=A16, scales_bf16=A16, y=A16, xq=A16,
                xs=A16, acc_out=None)

    def call(**kw):
        items = (_lib.ForwardItem * 2)(_lib.ForwardItem(**good), _lib.ForwardItem(**dict(good, **kw)))
        return L.s3d8_forward_batch(2, ctypes.addressof(items), None)

    assert call(x=None) == _lib.S3D8_ERR_INVALID_ARG
    assert call(xs=None) == _lib.S3D8_ERR_INVALID_ARG
    assert call(K=40) == _lib.S3D8_ERR_SHAPE
    assert call(x=A_ODD) == _lib.S3D8_ERR_ALIGN
    assert call(tiled=A_ODD) == _lib.S3D8_ERR_ALIGN
    assert call(tiled_bytes=0) == _lib.S3D8_ERR_INVALID_ARG
    assert ctypes.sizeof(_lib.ForwardItem) == 96


def test_encode_device_validation():
    L = _lib.lib()
    assert L.s3d8_encode_device(None, 3, 16, A16, A16, A16, None) == _lib.S3D8_ERR_INVALID_ARG
    assert L.s3d8_encode_device(A16, 3, 24, A16, A16, A16, None) == _lib.S3D8_ERR_SHAPE
    assert L.s3d8_encode_device(A16 + 2, 3, 16, A16, A16, A16, None) == _lib.S3D8_ERR_ALIGN
    assert L.s3d8_encode_device(A16, 3, 16, A16, A_ODD, A16, None) == _lib.S3D8_ERR_ALIGN
    assert L.s3d8_encode_device(A16, 0, 16, A16, A16, A16, None) == _lib.S3D8_ERR_INVALID_ARG
    assert L.s3d8_encode_device(A16, 1 << 20, 1 << 12, A16, A16, A16, None) == _lib.S3D8_ERR_SHAPE


def test_host_validation_errors():
    W = np.zeros((3, 16), np.float32)
    with pytest.raises(s3d8.S3D8Error) as e:
        s3d8.pack(np.zeros((3, 8), np.float32))
    assert e.value.code == _lib.S3D8_ERR_SHAPE
    with pytest.raises(s3d8.S3D8Error) as e:
        s3d8.pack(W, max_iters=-1)
    assert e.value.code == _lib.S3D8_ERR_INVALID_ARG
    bad = np.full((32, 3), 128, np.uint8)
    with pytest.raises(s3d8.S3D8Error) as e:
        s3d8.encode(W, bad)
    assert e.value.code == _lib.S3D8_ERR_INVALID_ARG and "127" in str(e.value)
    L = _lib.lib()
    assert L.s3d8_pack(None, 3, 16, 0, 1, 1, A16, A16, A16, None, None) == _lib.S3D8_ERR_INVALID_ARG
    assert L.s3d8_encode(W.ctypes.data, 3, 16, None, 1, A16, A16) == _lib.S3D8_ERR_INVALID_ARG


def test_last_error_cleared_by_success():
    W = np.zeros((3, 16), np.float32)
    with pytest.raises(s3d8.S3D8Error):
        s3d8.pack(np.zeros((3, 8), np.float32))
    assert _lib.lib().s3d8_last_error().decode() != ""
    s3d8.encode(W, np.ones((32, 3), np.uint8))
    assert _lib.lib().s3d8_last_error().decode() == ""


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(ImportError):
        _lib.lib()


def test_variant_entry_points_validation():
    """The format / output-type entry points reject unknown variants and
    validate like the entry points they extend, before any GPU work."""
    L = _lib.lib()

    def lin(fmt=0, out=0, **kw):
        a = dict(xq=A16, xs=A16, M=1, K=64, N=9, t=A16, C=A16, s=A16, y=A16, acc=None)
        a.update(kw)
        return L.s3d8_linear_ex(a["xq"], a["xs"], a["M"], a["K"], a["N"], a["t"], TB, a["C"], fmt, a["s"],
                                a["y"], out, a["acc"], None)

    assert lin(fmt=2) == _lib.S3D8_ERR_INVALID_ARG
    assert lin(fmt=-1) == _lib.S3D8_ERR_INVALID_ARG
    assert lin(out=2) == _lib.S3D8_ERR_INVALID_ARG
    assert "format" in L.s3d8_last_error().decode() or "output" in L.s3d8_last_error().decode()
    assert lin(fmt=1, out=1, y=None) == _lib.S3D8_ERR_INVALID_ARG
    assert lin(fmt=1, K=40) == _lib.S3D8_ERR_SHAPE
    assert lin(fmt=1, C=A16 + 2) == _lib.S3D8_ERR_ALIGN
    assert lin(out=1, t=A_ODD) == _lib.S3D8_ERR_ALIGN

    def fwd(fmt=0, out=0, **kw):
        a = dict(x=A16, M=1, K=64, N=9, t=A16, C=A16, s=A16, y=A16, xq=A16, xs=A16, acc=None)
        a.update(kw)
        return L.s3d8_forward_ex(a["x"], a["M"], a["K"], a["N"], a["t"], TB, a["C"], fmt, a["s"], a["y"], out,
                                 a["xq"], a["xs"], a["acc"], None)

    assert fwd(fmt=7) == _lib.S3D8_ERR_INVALID_ARG
    assert fwd(out=-1) == _lib.S3D8_ERR_INVALID_ARG
    assert fwd(fmt=1, x=None) == _lib.S3D8_ERR_INVALID_ARG
    assert fwd(fmt=1, out=1, x=A_ODD) == _lib.S3D8_ERR_ALIGN
    assert fwd(fmt=1, K=8) == _lib.S3D8_ERR_SHAPE

    def unf(fmt=0, out=0, **kw):
        a = dict(xq=A16, xs=A16, M=1, K=64, N=9, t=A16, C=A16, s=A16, y=A16, acc=None, ws=A16, wb=1 << 20)
        a.update(kw)
        return L.s3d8_linear_unfused_ex(a["xq"], a["xs"], a["M"], a["K"], a["N"], a["t"], TB, a["C"], fmt,
                                        a["s"], a["y"], out, a["acc"], a["ws"], a["wb"], None)

    assert unf(fmt=3) == _lib.S3D8_ERR_INVALID_ARG
    assert unf(out=5) == _lib.S3D8_ERR_INVALID_ARG
    assert unf(fmt=1, wb=16) == _lib.S3D8_ERR_INVALID_ARG
    assert unf(out=1, ws=None) == _lib.S3D8_ERR_INVALID_ARG

    assert L.s3d8_dequant_ex(A16, A16, 2, 9, 64, A16, None) == _lib.S3D8_ERR_INVALID_ARG
    assert L.s3d8_dequant_ex(A16, None, 1, 9, 64, A16, None) == _lib.S3D8_ERR_INVALID_ARG
    assert L.s3d8_dequant_ex(A16, A16 + 2, 1, 9, 64, A16, None) == _lib.S3D8_ERR_ALIGN
    assert L.s3d8_dequant_ex(A16, A16, 1, 9, 24, A16, None) == _lib.S3D8_ERR_SHAPE


def _splitk_bytes_closed_form(M, K, N, splits):
    """Two int32 counters per output tile (padded to 256 bytes) plus, per
    tile, `splits` slots of 4 waves x 3 RT accumulators x 64 lanes x 16
    int32; the largest need of the three tile heights (RT = 2, 4, 5 rows of
    32)."""
    T = -(-N // 3)
    KB = -(-K // 64)
    s = max(1, min(splits, KB))
    kbper = -(-KB // s)
    s = -(-KB // kbper)
    if M <= 16 or s == 1:
        return 0
    best = 0
    for rt in (2, 4, 5):
        tiles = -(-M // (32 * rt)) * -(-(-(-T // 16)) // 8)
        best = max(best, -(-(8 * tiles) // 256) * 256 + tiles * s * 4 * 3 * rt * 64 * 16 * 4)
    return best


@pytest.mark.parametrize("M,K,N,splits", [(1601, 5120, 1280, 4), (1601, 1280, 5120, 2), (2048, 4096, 14336, 3),
                                          (300, 1040, 772, 5), (17, 80, 50, 7), (33, 640, 97, 4),
                                          (33, 640, 97, 6), (1601, 5120, 1280, 1)])
def test_splitk_workspace_bytes(M, K, N, splits):
    L = _lib.lib()
    assert L.s3d8_splitk_workspace_bytes(M, K, N, splits) == _splitk_bytes_closed_form(M, K, N, splits)


def test_splitk_sizes_and_choice():
    L = _lib.lib()
    # worked case: the vision MLP down-projection at 1601 tokens takes
    # 64-row tiles (26 x 4 = 104 tiles of 64 rows x 384 channels, one round
    # on 256 CUs, against 52 tiles of 128 rows) and has 80 column blocks:
    # ceil(80/S) + 9 S is 89, 58 for S = 1, 2 and 3 x 104 tiles would not fit
    # one round, so 2 ranges; its workspace at 4 (RT = 5 needs the most:
    # 11 x 4 tiles)
    assert L.s3d8_splitk_auto(1601, 5120, 1280, 256) == 2
    assert L.s3d8_splitk_workspace_bytes(1601, 5120, 1280, 4) == 512 + 44 * 4 * 4 * 61440
    assert L.s3d8_splitk_auto(1601, 5120, 1280, 104) == 1  # 104 tiles fill every CU
    assert L.s3d8_splitk_auto(1601, 5120, 1280, 103) == 1
    assert L.s3d8_splitk_auto(1601, 1280, 5120, 256) == 1  # up-projection: 182 tiles
    assert L.s3d8_splitk_auto(2048, 4096, 14336, 256) == 1
    assert L.s3d8_splitk_auto(16, 5120, 1280, 256) == 1    # GEMV path
    assert L.s3d8_splitk_auto(17, 12800, 96, 256) == 5     # 200 blocks: 40 + 45 < 50 + 36
    assert L.s3d8_splitk_auto(17, 64 * 4000, 96, 256) == 16  # at most 16 ranges
    assert L.s3d8_splitk_auto(17, 256, 96, 256) == 1       # 4 blocks: no split
    assert L.s3d8_splitk_auto(0, 64, 9, 256) == -1
    assert L.s3d8_splitk_auto(1601, 5120, 1280, 0) == -1
    assert L.s3d8_splitk_workspace_bytes(16, 5120, 1280, 4) == 0
    assert L.s3d8_splitk_workspace_bytes(1601, 5120, 1280, 0) == -1
    assert L.s3d8_splitk_workspace_bytes(17, 80, 50, 1) == 0
    # ranges are rounded so that none is empty: 10 blocks in 6 requested
    # ranges become 5 ranges of 2
    assert L.s3d8_splitk_workspace_bytes(33, 640, 97, 6) == L.s3d8_splitk_workspace_bytes(33, 640, 97, 5)


def test_splitk_validation():
    L = _lib.lib()
    M, K, N = 1601, 5120, 1280
    need = L.s3d8_splitk_workspace_bytes(M, K, N, 4)

    def call(ws=A16, nbytes=need, splits=4, fmt=0, out=0, xq=A16, M=M, N=N):
        return L.s3d8_linear_splitk(xq, A16, M, K, N, A16, TB, A16, fmt, A16, A16, out, None, splits, ws, nbytes,
                                    None)

    assert call(splits=-1) == _lib.S3D8_ERR_INVALID_ARG
    assert call(ws=None) == _lib.S3D8_ERR_INVALID_ARG
    assert call(nbytes=need - 1) == _lib.S3D8_ERR_INVALID_ARG
    assert b"workspace" in L.s3d8_last_error()
    assert call(ws=A16 + 16) == _lib.S3D8_ERR_ALIGN
    assert call(xq=A_ODD) == _lib.S3D8_ERR_ALIGN
    assert call(fmt=2) == _lib.S3D8_ERR_INVALID_ARG
    assert call(out=5) == _lib.S3D8_ERR_INVALID_ARG
    assert call(N=3355443 * 3) == _lib.S3D8_ERR_SHAPE
    # partial sums over 2^31 bytes
    assert call(M=100000, N=12800, nbytes=1 << 40) == _lib.S3D8_ERR_SHAPE
    assert b"partial" in L.s3d8_last_error()
