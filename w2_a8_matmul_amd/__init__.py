"""S3D8 weight-decode-fused linear layer for AMD Instinct MI355X (gfx950).

Thin Python binding over the C ABI of ``libs3d8.so`` (``include/s3d8.h``):
argument marshalling only.  Host functions take numpy arrays; device
functions take torch tensors (device memory and the current HIP stream) and
run the library's HIP kernels.  There is no fallback path: if the library
is missing, importing ``w2_a8_matmul_amd._lib`` raises.

Format: the S3D8 storage format of "Llama-Mobile: Efficient 2.7-Bit
Quantization of VLMs" (Sec. 3.4, Eq. 1) with the byte layout of the blog
"11 billion parameters on a phone" ("Bit layout").  The device functions also
take 3D8 weights (``fmt="3d8"``: the table is int8 [256][3] signed
centroids indexed by the whole byte, the format the blog sets beside S3D8)
and write bf16 outputs (``out="bf16"``, as the blog's fused kernel does).
"""
from __future__ import annotations

import ctypes

import numpy as np

from ._lib import S3D8Error, call, lib  # noqa: F401

__all__ = [
    "S3D8Error", "num_triples", "packed_bytes", "format_bytes", "tiled_bytes", "pack", "encode",
    "tile", "quant_act", "linear", "linear_unfused", "unfused_workspace_bytes", "forward", "dequant",
    "PackedLinear", "hbm_read_probe", "mfma_rate_probe", "encode_device", "forward_batch",
    "linear_splitk", "splitk_auto", "splitk_workspace_bytes",
]


def _np_ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def num_triples(N: int) -> int:
    return int(lib().s3d8_num_triples(N))


def packed_bytes(N: int, K: int) -> int:
    return int(lib().s3d8_packed_bytes(N, K))


def format_bytes(N: int, K: int) -> int:
    return int(lib().s3d8_format_bytes(N, K))


def tiled_bytes(N: int, K: int) -> int:
    return int(lib().s3d8_tiled_bytes(N, K))


# ------------------------------------------------------------------ host
def pack(W, seed: int = 1, max_iters: int = 50, num_threads: int = 0, return_stats: bool = False):
    """Fit centroids (k-means++ / Lloyd-Max) and encode W (fp32 [N][K]).

    Returns (centroids uint8 [32][3], scales_bf16 uint16 [3T], packed uint8
    [T][K]) and, with ``return_stats``, also (distortion per iteration,
    iterations)."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    N, K = W.shape
    T = num_triples(N)
    C = np.empty((32, 3), np.uint8)
    scales = np.empty((3 * T,), np.uint16)
    packed = np.empty((T, K), np.uint8)
    dist = np.zeros((max(max_iters, 0) + 1,), np.float64)
    iters = ctypes.c_int32(0)
    call("s3d8_pack", _np_ptr(W), N, K, seed, max_iters, num_threads, _np_ptr(C), _np_ptr(scales),
         _np_ptr(packed), _np_ptr(dist), ctypes.byref(iters))
    if return_stats:
        return C, scales, packed, dist[: iters.value + 1].copy(), iters.value
    return C, scales, packed


def encode(W, centroids, num_threads: int = 0):
    """Frozen-centroid encode: returns (scales_bf16 [3T], packed [T][K])."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    C = np.ascontiguousarray(centroids, dtype=np.uint8)
    N, K = W.shape
    T = num_triples(N)
    scales = np.empty((3 * T,), np.uint16)
    packed = np.empty((T, K), np.uint8)
    call("s3d8_encode", _np_ptr(W), N, K, _np_ptr(C), num_threads, _np_ptr(scales), _np_ptr(packed))
    return scales, packed


# ------------------------------------------------------------------ device
def _torch():
    import torch
    return torch


def _stream(t) -> int:
    torch = _torch()
    return torch.cuda.current_stream(t.device).cuda_stream


def _dev_check(t, dtype, name, device=None, numel=None, min_numel=None):
    """A device tensor argument: torch tensor on the GPU (on `device` when
    given), of `dtype`, contiguous, and with exactly `numel` (or at least
    `min_numel`) elements when given.  Outputs are checked with numel, so the
    kernels never write past a caller-supplied buffer."""
    torch = _torch()
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError(f"{name} must be a CUDA/HIP torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must have dtype {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the other arguments on {device}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must have {numel} elements, got {t.numel()}")
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError(f"{name} must have at least {min_numel} elements, got {t.numel()}")


def quant_act(x, xq=None, xs=None):
    """Per-token INT8 quantisation of fp32 x [M][K] on the GPU: (xq, xs)."""
    torch = _torch()
    _dev_check(x, torch.float32, "x")
    M, K = x.shape
    xq, xs = _codes_out(xq, xs, M, K, x.device)
    with torch.cuda.device(x.device):
        call("s3d8_quant_act", x.data_ptr(), M, K, xq.data_ptr(), xs.data_ptr(), _stream(x))
    return xq, xs


def tile(packed, N: int, tiled=None):
    """Re-lay a device packed matrix [T][K] into the tiled layout read by
    linear/forward (done once per matrix)."""
    torch = _torch()
    _dev_check(packed, torch.uint8, "packed")
    T, K = packed.shape
    if T != num_triples(N):
        raise ValueError("packed rows do not match N")
    if tiled is None:
        tiled = torch.empty((tiled_bytes(N, K),), dtype=torch.uint8, device=packed.device)
    _dev_check(tiled, torch.uint8, "tiled", packed.device, min_numel=tiled_bytes(N, K))
    with torch.cuda.device(packed.device):
        call("s3d8_tile", packed.data_ptr(), N, K, tiled.data_ptr(), _stream(packed))
    return tiled


def _scales_view(scales):
    torch = _torch()
    if scales.dtype in (torch.bfloat16, torch.uint16):
        scales = scales.view(torch.int16)
    _dev_check(scales, torch.int16, "scales")
    return scales


_FORMATS = {"s3d8": 0, "3d8": 1}
_OUTS = {"f32": 0, "bf16": 1}


def _variant(fmt: str, out: str = "f32"):
    if fmt not in _FORMATS or out not in _OUTS:
        raise ValueError(f"fmt must be one of {list(_FORMATS)}, out one of {list(_OUTS)}")
    return _FORMATS[fmt], _OUTS[out]


def _table_view(table, fmt: str):
    """S3D8: uint8 [32][3] centroids; 3D8: int8 [256][3] signed table (uint8 views accepted)."""
    torch = _torch()
    if fmt == "3d8" and table.dtype == torch.int8:
        table = table.view(torch.uint8)
    _dev_check(table, torch.uint8, "centroids" if fmt == "s3d8" else "table")
    if table.numel() != (96 if fmt == "s3d8" else 768):
        raise ValueError("table size does not match the format")
    return table


def _check_weights(tiled, centroids, scales, N, K, fmt: str = "s3d8", device=None):
    torch = _torch()
    _dev_check(tiled, torch.uint8, "tiled", device)
    table = _table_view(centroids, fmt)
    _dev_check(table, torch.uint8, "centroids", device)
    _dev_check(scales, torch.int16, "scales", device)
    T = num_triples(N)
    if tiled.numel() < tiled_bytes(N, K) or scales.numel() < 3 * T:
        raise ValueError("tiled / centroids / scales do not match (N, K)")


def _y_out(y, M, N, out, device):
    """The output buffer: a new one, or a caller's of the right type and size."""
    torch = _torch()
    dtype = torch.float32 if out == "f32" else torch.bfloat16
    if y is None:
        return torch.empty((M, N), dtype=dtype, device=device)
    _dev_check(y, dtype, "y", device, numel=M * N)
    return y


def _acc_out(acc, want, M, N, device):
    torch = _torch()
    if acc is None:
        return torch.empty((M, N), dtype=torch.int32, device=device) if want else None
    _dev_check(acc, torch.int32, "acc", device, numel=M * N)
    return acc


def _codes_out(xq, xs, M, K, device):
    """Activation codes and scales written by quant_act / forward."""
    torch = _torch()
    if xq is None:
        xq = torch.empty((M, K), dtype=torch.int8, device=device)
    if xs is None:
        xs = torch.empty((M,), dtype=torch.float32, device=device)
    _dev_check(xq, torch.int8, "xq", device, numel=M * K)
    _dev_check(xs, torch.float32, "xs", device, numel=M)
    return xq, xs


def linear(xq, xs, tiled, centroids, scales, N: int, y=None, acc=None, return_acc: bool = False,
           fmt: str = "s3d8", out: str = "f32"):
    """Fused S3D8 (or 3D8) linear on pre-quantised activations: y [M][N],
    fp32 or bf16 (and the INT32 accumulators)."""
    torch = _torch()
    f, o = _variant(fmt, out)
    _dev_check(xq, torch.int8, "xq")
    M, K = xq.shape
    _dev_check(xs, torch.float32, "xs", xq.device, min_numel=M)
    scales = _scales_view(scales)
    _check_weights(tiled, centroids, scales, N, K, fmt, xq.device)
    y = _y_out(y, M, N, out, xq.device)
    acc = _acc_out(acc, return_acc, M, N, xq.device)
    with torch.cuda.device(xq.device):
        args = (xq.data_ptr(), xs.data_ptr(), M, K, N, tiled.data_ptr(), tiled.numel(), centroids.data_ptr())
        tail = (acc.data_ptr() if acc is not None else None, _stream(xq))
        if f == 0 and o == 0:
            call("s3d8_linear", *args, scales.data_ptr(), y.data_ptr(), *tail)
        else:
            call("s3d8_linear_ex", *args, f, scales.data_ptr(), y.data_ptr(), o, *tail)
    if return_acc:
        return y, acc
    return y


def unfused_workspace_bytes(N: int, K: int) -> int:
    return int(lib().s3d8_unfused_workspace_bytes(N, K))


def linear_unfused(xq, xs, tiled, centroids, scales, N: int, workspace=None, y=None, acc=None,
                   return_acc: bool = False, fmt: str = "s3d8", out: str = "f32"):
    """Same result as ``linear``: the matrix is decoded once into an INT8
    workspace (allocated here unless given), then an INT8 GEMM runs on it."""
    torch = _torch()
    f, o = _variant(fmt, out)
    _dev_check(xq, torch.int8, "xq")
    M, K = xq.shape
    _dev_check(xs, torch.float32, "xs", xq.device, min_numel=M)
    scales = _scales_view(scales)
    _check_weights(tiled, centroids, scales, N, K, fmt, xq.device)
    wbytes = unfused_workspace_bytes(N, K)
    if workspace is None:
        workspace = torch.empty((wbytes,), dtype=torch.int8, device=xq.device)
    _dev_check(workspace, torch.int8, "workspace", xq.device, min_numel=wbytes)
    y = _y_out(y, M, N, out, xq.device)
    acc = _acc_out(acc, return_acc, M, N, xq.device)
    with torch.cuda.device(xq.device):
        args = (xq.data_ptr(), xs.data_ptr(), M, K, N, tiled.data_ptr(), tiled.numel(), centroids.data_ptr())
        tail = (acc.data_ptr() if acc is not None else None, workspace.data_ptr(), workspace.numel(),
                _stream(xq))
        if f == 0 and o == 0:
            call("s3d8_linear_unfused", *args, scales.data_ptr(), y.data_ptr(), *tail)
        else:
            call("s3d8_linear_unfused_ex", *args, f, scales.data_ptr(), y.data_ptr(), o, *tail)
    if return_acc:
        return y, acc
    return y


def splitk_auto(M: int, K: int, N: int, num_cus: int) -> int:
    return int(lib().s3d8_splitk_auto(M, K, N, num_cus))


def splitk_workspace_bytes(M: int, K: int, N: int, splits: int) -> int:
    return int(lib().s3d8_splitk_workspace_bytes(M, K, N, splits))


def linear_splitk(xq, xs, tiled, centroids, scales, N: int, splits: int = 0, workspace=None, y=None, acc=None,
                  return_acc: bool = False, fmt: str = "s3d8", out: str = "f32"):
    """Same result as ``linear``, with the fused GEMM's input columns split
    into ``splits`` ranges whose INT32 partial sums are added before the
    epilogue (0: the library's choice for this GPU).  The workspace holds the
    partial sums and per-tile counters; it is allocated here, zero-filled,
    unless given (a given one must have been zero-filled before its first
    use; each call leaves it ready for the next)."""
    torch = _torch()
    f, o = _variant(fmt, out)
    _dev_check(xq, torch.int8, "xq")
    M, K = xq.shape
    _dev_check(xs, torch.float32, "xs", xq.device, min_numel=M)
    scales = _scales_view(scales)
    _check_weights(tiled, centroids, scales, N, K, fmt, xq.device)
    if splits == 0:
        splits = splitk_auto(M, K, N, torch.cuda.get_device_properties(xq.device).multi_processor_count)
    if splits < 1:
        raise ValueError("splits must be 0 (automatic) or positive")
    wbytes = splitk_workspace_bytes(M, K, N, splits)
    if workspace is None:
        workspace = torch.zeros((max(wbytes, 1),), dtype=torch.uint8, device=xq.device)
    _dev_check(workspace, torch.uint8, "workspace", xq.device, min_numel=wbytes)
    y = _y_out(y, M, N, out, xq.device)
    acc = _acc_out(acc, return_acc, M, N, xq.device)
    with torch.cuda.device(xq.device):
        call("s3d8_linear_splitk", xq.data_ptr(), xs.data_ptr(), M, K, N, tiled.data_ptr(), tiled.numel(),
             centroids.data_ptr(), f, scales.data_ptr(), y.data_ptr(), o,
             acc.data_ptr() if acc is not None else None, splits, workspace.data_ptr(), workspace.numel(),
             _stream(xq))
    if return_acc:
        return y, acc
    return y


def forward(x, tiled, centroids, scales, N: int, y=None, xq=None, xs=None, acc=None,
            return_all: bool = False, fmt: str = "s3d8", out: str = "f32"):
    """The whole path from fp32 x [M][K]: quantise and apply the S3D8 (or
    3D8) linear (one kernel launch for M <= 4).  Returns y, or (y, xq, xs,
    acc) with ``return_all``."""
    torch = _torch()
    f, o = _variant(fmt, out)
    _dev_check(x, torch.float32, "x")
    scales = _scales_view(scales)
    M, K = x.shape
    _check_weights(tiled, centroids, scales, N, K, fmt, x.device)
    y = _y_out(y, M, N, out, x.device)
    xq, xs = _codes_out(xq, xs, M, K, x.device)
    acc = _acc_out(acc, return_all, M, N, x.device)
    with torch.cuda.device(x.device):
        tail = (xq.data_ptr(), xs.data_ptr(), acc.data_ptr() if acc is not None else None, _stream(x))
        if f == 0 and o == 0:
            call("s3d8_forward", x.data_ptr(), M, K, N, tiled.data_ptr(), tiled.numel(), centroids.data_ptr(),
                 scales.data_ptr(), y.data_ptr(), *tail)
        else:
            call("s3d8_forward_ex", x.data_ptr(), M, K, N, tiled.data_ptr(), tiled.numel(), centroids.data_ptr(),
                 f, scales.data_ptr(), y.data_ptr(), o, *tail)
    if return_all:
        return y, xq, xs, acc
    return y


def forward_batch(items, return_all: bool = False):
    """Several ``forward`` calls in one go (one kernel launch when they fit
    the streaming GEMV together, see s3d8_forward_batch).  ``items`` is a
    list of dicts with keys x, tiled, centroids, scales, N and optionally y,
    xq, xs, acc.  Returns the list of y (or of (y, xq, xs, acc) tuples with
    ``return_all``)."""
    torch = _torch()
    arr = (_lib.ForwardItem * max(1, len(items)))()
    outs = []
    dev = None
    for i, it in enumerate(items):
        x = it["x"]
        _dev_check(x, torch.float32, "x")
        scales = _scales_view(it["scales"])
        M, K = x.shape
        N = int(it["N"])
        if dev is None:
            dev = x.device
        elif x.device != dev:
            raise ValueError("all items must be on one device")
        _check_weights(it["tiled"], it["centroids"], scales, N, K, device=dev)
        y = _y_out(it.get("y"), M, N, "f32", dev)
        xq, xs = _codes_out(it.get("xq"), it.get("xs"), M, K, dev)
        acc = _acc_out(it.get("acc"), return_all, M, N, dev)
        arr[i] = _lib.ForwardItem(x.data_ptr(), M, K, N, it["tiled"].data_ptr(), it["tiled"].numel(),
                                  it["centroids"].data_ptr(), scales.data_ptr(), y.data_ptr(), xq.data_ptr(),
                                  xs.data_ptr(), acc.data_ptr() if acc is not None else None)
        outs.append((y, xq, xs, acc, x, scales))
    if items:
        with torch.cuda.device(dev):
            call("s3d8_forward_batch", len(items), ctypes.addressof(arr), _stream(items[0]["x"]))
    if return_all:
        return [o[:4] for o in outs]
    return [o[0] for o in outs]


def encode_device(W, centroids):
    """Frozen-centroid encode on the GPU (same results as ``encode``):
    returns (scales bf16 bits as int16 [3T], packed uint8 [T][K])."""
    torch = _torch()
    _dev_check(W, torch.float32, "W")
    _dev_check(centroids, torch.uint8, "centroids")
    N, K = W.shape
    T = num_triples(N)
    scales = torch.empty((3 * T,), dtype=torch.int16, device=W.device)
    packed = torch.empty((T, K), dtype=torch.uint8, device=W.device)
    with torch.cuda.device(W.device):
        call("s3d8_encode_device", W.data_ptr(), N, K, centroids.data_ptr(), scales.data_ptr(), packed.data_ptr(),
             _stream(W))
    return scales, packed


def dequant(packed, centroids, N: int, w=None, fmt: str = "s3d8"):
    """Standalone decode to channel-INT8: w int8 [N][K]."""
    torch = _torch()
    f, _ = _variant(fmt)
    _dev_check(packed, torch.uint8, "packed")
    centroids = _table_view(centroids, fmt)
    T, K = packed.shape
    if T != num_triples(N):
        raise ValueError("packed rows do not match N")
    if w is None:
        w = torch.empty((N, K), dtype=torch.int8, device=packed.device)
    _dev_check(centroids, torch.uint8, "centroids", packed.device)
    _dev_check(w, torch.int8, "w", packed.device, numel=N * K)
    with torch.cuda.device(packed.device):
        if f == 0:
            call("s3d8_dequant", packed.data_ptr(), centroids.data_ptr(), N, K, w.data_ptr(), _stream(packed))
        else:
            call("s3d8_dequant_ex", packed.data_ptr(), centroids.data_ptr(), f, N, K, w.data_ptr(),
                 _stream(packed))
    return w


def mfma_rate_probe(iters: int, workgroups: int, v: int = 1, out=None, device="cuda"):
    """Matrix-core rate probe (a measurement utility): `workgroups` x 4
    waves each run `iters` rounds of four independent 32x32x32 INT8 MFMAs;
    every word of out (int32 [256 * workgroups]) becomes 2048 v^2 iters
    (mod 2^32).  Returns (out, integer operations performed)."""
    torch = _torch()
    if out is None:
        out = torch.empty((256 * workgroups,), dtype=torch.int32, device=device)
    _dev_check(out, torch.int32, "out")
    if out.numel() < 256 * workgroups:
        raise ValueError("out must hold 256 * workgroups int32")
    with torch.cuda.device(out.device):
        call("s3d8_mfma_rate_probe", iters, workgroups, v, out.data_ptr(), _stream(out))
    return out, workgroups * 4 * 4 * iters * 65536


def hbm_read_probe(buf, workgroups: int, out=None):
    """Memory read probe (a measurement utility): `workgroups` workgroups of
    256 threads stream the bytes of the device tensor `buf` (a multiple of 16
    bytes) and workgroup w stores the XOR of the 32-bit words it read into
    out[w] (uint32 as int32 [workgroups]).  Returns out."""
    torch = _torch()
    if not isinstance(buf, torch.Tensor) or buf.device.type != "cuda" or not buf.is_contiguous():
        raise TypeError("buf must be a contiguous CUDA/HIP torch tensor")
    if out is None:
        out = torch.empty((workgroups,), dtype=torch.int32, device=buf.device)
    _dev_check(out, torch.int32, "out", buf.device, min_numel=workgroups)
    nbytes = buf.numel() * buf.element_size()
    with torch.cuda.device(buf.device):
        call("s3d8_hbm_read_probe", buf.data_ptr(), nbytes, workgroups, out.data_ptr(), _stream(buf))
    return out


class PackedLinear:
    """An S3D8 weight matrix resident in device memory, in the tiled layout."""

    def __init__(self, centroids, scales, packed, N: int, device="cuda"):
        torch = _torch()
        self.N = int(N)
        self.K = int(packed.shape[1])
        self.centroids = torch.as_tensor(np.ascontiguousarray(centroids, np.uint8)).to(device)
        self.scales = torch.as_tensor(np.ascontiguousarray(scales, np.uint16).view(np.int16)).to(device)
        packed_dev = torch.as_tensor(np.ascontiguousarray(packed, np.uint8)).to(device)
        self.tiled = tile(packed_dev, self.N)

    @classmethod
    def from_weights(cls, W, seed: int = 1, max_iters: int = 50, device="cuda"):
        C, s, p = pack(W, seed=seed, max_iters=max_iters)
        return cls(C, s, p, W.shape[0], device)

    def __call__(self, x):
        return forward(x, self.tiled, self.centroids, self.scales, self.N)
