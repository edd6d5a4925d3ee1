"""ctypes view of libs3d8.so: the symbols and signatures of include/s3d8.h.

Loading fails loudly (ImportError) when the library has not been built;
there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

# S3D8_LIB selects another build of the library (e.g. the sanitizer build of
# the host code, build.py --sanitize); by default the in-tree libs3d8.so
LIB_PATH = os.environ.get("S3D8_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libs3d8.so")

S3D8_OK = 0
S3D8_ERR_INVALID_ARG = 1
S3D8_ERR_SHAPE = 2
S3D8_ERR_ALIGN = 3
S3D8_ERR_HIP = 4
S3D8_ERR_NOMEM = 5
S3D8_ERR_DEVICE = 6
S3D8_NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_U64 = ctypes.c_uint64

# name -> (restype, argtypes); mirrors include/s3d8.h
SIGNATURES = {
    "s3d8_version": (_I32, []),
    "s3d8_num_triples": (_I64, [_I64]),
    "s3d8_packed_bytes": (_I64, [_I64, _I64]),
    "s3d8_format_bytes": (_I64, [_I64, _I64]),
    "s3d8_last_error": (ctypes.c_char_p, []),
    "s3d8_pack": (_I32, [_P, _I64, _I64, _U64, _I32, _I32, _P, _P, _P, _P, _P]),
    "s3d8_encode": (_I32, [_P, _I64, _I64, _P, _I32, _P, _P]),
    "s3d8_quant_act": (_I32, [_P, _I64, _I64, _P, _P, _P]),
    "s3d8_tiled_bytes": (_I64, [_I64, _I64]),
    "s3d8_tile": (_I32, [_P, _I64, _I64, _P, _P]),
    "s3d8_linear": (_I32, [_P, _P, _I64, _I64, _I64, _P, _I64, _P, _P, _P, _P, _P]),
    "s3d8_forward": (_I32, [_P, _I64, _I64, _I64, _P, _I64, _P, _P, _P, _P, _P, _P, _P]),
    "s3d8_dequant": (_I32, [_P, _P, _I64, _I64, _P, _P]),
    "s3d8_unfused_workspace_bytes": (_I64, [_I64, _I64]),
    "s3d8_linear_unfused": (_I32, [_P, _P, _I64, _I64, _I64, _P, _I64, _P, _P, _P, _P, _P, _I64, _P]),
    "s3d8_forward_batch": (_I32, [_I32, _P, _P]),
    "s3d8_encode_device": (_I32, [_P, _I64, _I64, _P, _P, _P, _P]),
    "s3d8_linear_ex": (_I32, [_P, _P, _I64, _I64, _I64, _P, _I64, _P, _I32, _P, _P, _I32, _P, _P]),
    "s3d8_forward_ex": (_I32, [_P, _I64, _I64, _I64, _P, _I64, _P, _I32, _P, _P, _I32, _P, _P, _P, _P]),
    "s3d8_linear_unfused_ex": (_I32, [_P, _P, _I64, _I64, _I64, _P, _I64, _P, _I32, _P, _P, _I32, _P, _P, _I64, _P]),
    "s3d8_dequant_ex": (_I32, [_P, _P, _I32, _I64, _I64, _P, _P]),
    "s3d8_mfma_rate_probe": (_I32, [_I32, _I32, _I32, _P, _P]),
    "s3d8_hbm_read_probe": (_I32, [_P, _I64, _I32, _P, _P]),
    "s3d8_linear_unfused_noalloc": (_I32, [_P, _P, _I64, _I64, _I64, _P, _I64, _P, _P, _P, _P, _P]),
    "s3d8_linear_splitk": (_I32, [_P, _P, _I64, _I64, _I64, _P, _I64, _P, _I32, _P, _P, _I32, _P, _I32, _P, _I64,
                                  _P]),
    "s3d8_splitk_auto": (_I32, [_I64, _I64, _I64, _I32]),
    "s3d8_splitk_workspace_bytes": (_I64, [_I64, _I64, _I64, _I32]),
}


class ForwardItem(ctypes.Structure):
    """s3d8_forward_item of include/s3d8.h (all members 8 bytes wide)."""
    _fields_ = [("x", _P), ("M", _I64), ("K", _I64), ("N", _I64), ("tiled", _P), ("tiled_bytes", _I64),
                ("centroids", _P), ("scales_bf16", _P), ("y", _P), ("xq", _P), ("xs", _P), ("acc_out", _P)]

_lib = None


class S3D8Error(RuntimeError):
    def __init__(self, code: int, func: str, msg: str):
        super().__init__(f"{func} failed with status {code}: {msg}")
        self.code = code


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                              "or python w2_a8_matmul_amd/build.py")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(handle, name)
            f.restype = res
            f.argtypes = args
        _lib = handle
    return _lib


def check(code: int, func: str) -> None:
    if code != S3D8_OK:
        msg = lib().s3d8_last_error()
        raise S3D8Error(code, func, msg.decode() if msg else "")


def call(name: str, *args) -> None:
    check(getattr(lib(), name)(*args), name)
