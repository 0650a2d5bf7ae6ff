"""ctypes binding of libbsa.so (argument marshalling only).

Every computation runs in the library's HIP kernels.  PyTorch supplies device
memory (outputs and workspaces are torch tensors) and the current stream.
The binding raises when the library is missing: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libbsa.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "bsa.h")

BSA_OK, BSA_ERR_INVALID_ARG, BSA_ERR_UNSUPPORTED, BSA_ERR_WORKSPACE, BSA_ERR_HIP = range(5)
BSA_BF16, BSA_FP32 = 0, 1
BSA_WS_ESTIMATE, BSA_WS_FORWARD, BSA_WS_BACKWARD, BSA_WS_SELECT_FROM_MASS, BSA_WS_STRUCTURED = 0, 1, 2, 3, 4
BSA_WS_ESTIMATE_HIER = 5
(BSA_PATTERN_DENSE, BSA_PATTERN_SPATIAL, BSA_PATTERN_TEMPORAL, BSA_PATTERN_DIAGONAL, BSA_PATTERN_MULTI_DIAGONAL,
 BSA_PATTERN_STRIPES) = range(6)


class BsaShape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("N", ctypes.c_int32), ("D", ctypes.c_int32),
                ("block", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class BsaCsr(ctypes.Structure):
    _fields_ = [("row_ptr", ctypes.c_void_p), ("col_idx", ctypes.c_void_p), ("capacity", ctypes.c_int64)]


class BsaPatternParams(ctypes.Structure):
    _fields_ = [("prefix_tokens", ctypes.c_int32), ("frame_tokens", ctypes.c_int32), ("band", ctypes.c_int32),
                ("period", ctypes.c_int32), ("stripes", ctypes.c_void_p), ("n_stripes", ctypes.c_int32)]


class BsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Load libbsa.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m block_sparse_attention_16_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    L.bsa_workspace_size.argtypes = [P(BsaShape), i32, i64]
    L.bsa_workspace_size.restype = sz
    L.bsa_estimate_mask.argtypes = [P(BsaShape), vp, vp, f32, f32, P(BsaCsr), i32, P(BsaCsr), vp, sz, vp]
    L.bsa_estimate_mask.restype = i32
    L.bsa_estimate_mask_hierarchical.argtypes = [P(BsaShape), vp, vp, f32, f32, P(BsaCsr), i32, i32, P(BsaCsr), vp,
                                                 sz, vp]
    L.bsa_estimate_mask_hierarchical.restype = i32
    L.bsa_select_from_mass.argtypes = [P(BsaShape), P(BsaCsr), vp, f32, i32, P(BsaCsr), vp, sz, vp]
    L.bsa_select_from_mass.restype = i32
    L.bsa_select_from_mass_noalloc.argtypes = [P(BsaShape), P(BsaCsr), vp, f32, i32, P(BsaCsr), vp]
    L.bsa_select_from_mass_noalloc.restype = i32
    L.bsa_structured_mask.argtypes = [P(BsaShape), vp, P(BsaPatternParams), P(BsaCsr), vp, sz, vp]
    L.bsa_structured_mask.restype = i32
    L.bsa_permute_rows.argtypes = [i64, i32, i32, vp, vp, i32, vp, vp]
    L.bsa_permute_rows.restype = i32
    L.bsa_forward.argtypes = [P(BsaShape), vp, vp, vp, f32, P(BsaCsr), vp, vp, vp, vp, vp, sz, vp]
    L.bsa_forward.restype = i32
    L.bsa_backward.argtypes = [P(BsaShape), vp, vp, vp, vp, vp, vp, vp, f32, P(BsaCsr), vp, vp, vp, vp, sz, vp]
    L.bsa_backward.restype = i32
    L.bsa_status_string.argtypes = [i32]
    L.bsa_status_string.restype = ctypes.c_char_p
    L.bsa_last_error.argtypes = []
    L.bsa_last_error.restype = ctypes.c_char_p
    L.bsa_version.argtypes = []
    L.bsa_version.restype = i32
    _lib = L
    return L


def header_functions() -> list[str]:
    """Names of the functions declared in include/bsa.h."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(bsa_\w+)\s*\(", text, flags=re.M)))


def check(status: int, what: str) -> None:
    if status != BSA_OK:
        L = load()
        msg = L.bsa_last_error().decode()
        raise BsaError(status, f"{what}: {L.bsa_status_string(status).decode()}: {msg}")
