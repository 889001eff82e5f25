"""ctypes declarations of the C ABI in include/tr_sparseconv.h.

The library is loaded after torch so that both use the one HIP runtime torch
has already mapped into the process. There is no fallback: if the HIP library
is not built, loading raises.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (maps the HIP runtime first)

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtr_sparseconv.so")

OK = 0
ERR_INVALID_ARG = -1
ERR_COORD_RANGE = -2
ERR_DUPLICATE = -3
ERR_CAPACITY = -4
ERR_WORKSPACE = -5
ERR_UNSUPPORTED = -6
ERR_HIP = -7
STATUS_NAMES = {OK: "OK", ERR_INVALID_ARG: "INVALID_ARG", ERR_COORD_RANGE: "COORD_RANGE",
                ERR_DUPLICATE: "DUPLICATE", ERR_CAPACITY: "CAPACITY", ERR_WORKSPACE: "WORKSPACE",
                ERR_UNSUPPORTED: "UNSUPPORTED", ERR_HIP: "HIP"}

F32 = 0
BF16 = 1
F16 = 2

ACT_NONE = 0
ACT_RELU = 1
ACT_SILU = 2

# (name, restype, argtypes) of every exported symbol.
_P = ctypes.c_void_p
_PP = ctypes.POINTER(ctypes.c_void_p)
_I = ctypes.c_int
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
SIGNATURES = [
    ("tr_sparseconv_version", _I, []),
    ("tr_sparseconv_last_error", ctypes.c_char_p, []),
    ("tr_sparseconv_hash_workspace_bytes", _SZ, [_I64]),
    ("tr_sparseconv_build_hash", _I, [_P, _I64, _P, _SZ, _P, _PP]),
    ("tr_sparseconv_hash_grid_workspace_bytes", _SZ, [_I64, _I, _I]),
    ("tr_sparseconv_build_hash_grid", _I, [_P, _I64, _I, _I, _P, _SZ, _P, _PP]),
    ("tr_sparseconv_status", _I, [_P, _P]),
    ("tr_sparseconv_hash_size", _I64, [_P]),
    ("tr_sparseconv_hash_lookup", _I, [_P, _P, _I64, _P, _P]),
    ("tr_sparseconv_hash_sorted_rows", _I, [_P, _P, _P]),
    ("tr_sparseconv_hash_destroy", None, [_P]),
    ("tr_sparseconv_kmap_workspace_bytes", _SZ, [_I64]),
    ("tr_sparseconv_build_kernel_map", _I, [_P, _P, _P, _SZ, _P, _PP]),
    ("tr_sparseconv_kmap_destroy", None, [_P]),
    ("tr_sparseconv_forward_workspace_bytes", _SZ, [_I, _I, _I]),
    ("tr_sparseconv_forward", _I, [_P, _P, _P, _P, _I, _I, _I, _P, _SZ, _P]),
    ("tr_sparseconv_forward_noalloc", _I, [_P, _P, _P, _P, _I, _I, _I, _P]),
    ("tr_sparseconv_packed_weights_bytes", _SZ, [_I, _I, _I]),
    ("tr_sparseconv_pack_weights", _I, [_P, _I, _I, _I, _P, _SZ, _P]),
    ("tr_sparseconv_forward_packed", _I, [_P, _P, _P, _P, _I, _I, _I, _P]),
    ("tr_sparseconv_forward_fused", _I, [_P, _P, _I, _P, _I, _P, _I, _P, _P, _I, _I, _I, _P]),
    ("tr_sparseconv_pack_weights_dgrad", _I, [_P, _I, _I, _I, _P, _SZ, _P]),
    ("tr_sparseconv_backward_data", _I, [_P, _P, _I, _P, _I, _P, _I, _I, _I, _P]),
    ("tr_sparseconv_backward_weights_workspace_bytes", _SZ, [_I64, _I, _I, _I]),
    ("tr_sparseconv_backward_weights", _I, [_P, _P, _P, _P, _I, _I, _I, _P, _SZ, _P]),
    ("tr_sparseconv_level_workspace_bytes", _SZ, [_I64]),
    ("tr_sparseconv_downsample", _I, [_P, _P, _P, _I64, _P, _SZ, _P, ctypes.POINTER(ctypes.c_int64)]),
    ("tr_sparseconv_subdivide", _I, [_P, _I64, _P, _P, _P, _I64, _P, _SZ, _P, ctypes.POINTER(ctypes.c_int64)]),
    ("tr_sparseconv_channel2spatial", _I, [_P, _I64, _P, _P, _I, _I, _P]),
    ("tr_sparseconv_spatial2channel", _I, [_P, _I64, _P, _P, _I, _I, _P]),
    ("tr_sparseconv_ceiling_mfma_flops", _I64, [_I, _I]),
    ("tr_sparseconv_ceiling_mfma", _I, [_P, _I, _I, _P]),
    ("tr_sparseconv_ceiling_copy", _I, [_P, _P, _SZ, _I, _P]),
]

_lib = None


class TrSparseConvError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(code, code)}: {message}")
        self.code = code


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run "
                              "`python -m submanifold_sparse_conv_amd.build` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        for name, res, args in SIGNATURES:
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def check(code: int) -> None:
    if code != OK:
        msg = lib().tr_sparseconv_last_error()
        raise TrSparseConvError(code, msg.decode() if msg else "")
