"""ctypes declarations of the libdeformagg C ABI (include/deformagg.h, include/dcn.h).

Only marshalling lives here.  Loading fails loudly when the library has not
been built: there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import List

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libdeformagg.so")
HEADER_PATH = os.path.join(os.path.dirname(PKG_DIR), "include", "deformagg.h")
HEADER_PATHS = [HEADER_PATH, os.path.join(os.path.dirname(PKG_DIR), "include", "dcn.h")]

DA_OK, DA_ERR_INVALID_ARG, DA_ERR_UNSUPPORTED, DA_ERR_HIP = 0, 1, 2, 3
DA_F32, DA_BF16, DA_F16 = 0, 1, 2
DA_FLAG_SLICES_ALWAYS, DA_FLAG_SLICES_NEVER, DA_FLAG_BWD_REGATHER, DA_FLAG_BWD_ROW_ORDER = \
    1, 2, 4, 8
DA_FLAG_DETERMINISTIC = 16
DA_NOALLOC_SCRATCH_BYTES = 96 << 20


class DAProblem(ctypes.Structure):
    _fields_ = [
        ("bs", ctypes.c_int64),
        ("num_feat", ctypes.c_int64),
        ("num_embeds", ctypes.c_int64),
        ("num_anchors", ctypes.c_int64),
        ("num_pts", ctypes.c_int64),
        ("num_cams", ctypes.c_int64),
        ("num_scale", ctypes.c_int64),
        ("num_groups", ctypes.c_int64),
        ("feat_dtype", ctypes.c_int32),
        ("flags", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


class DCNProblem(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int64),
        ("height", ctypes.c_int64),
        ("width", ctypes.c_int64),
        ("channels", ctypes.c_int64),
        ("groups", ctypes.c_int64),
        ("kernel_h", ctypes.c_int32), ("kernel_w", ctypes.c_int32),
        ("stride_h", ctypes.c_int32), ("stride_w", ctypes.c_int32),
        ("pad_h", ctypes.c_int32), ("pad_w", ctypes.c_int32),
        ("dilation_h", ctypes.c_int32), ("dilation_w", ctypes.c_int32),
        ("in_dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32),
        ("flags", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


class DAPackProblem(ctypes.Structure):
    _fields_ = [
        ("bs", ctypes.c_int64),
        ("num_cams", ctypes.c_int64),
        ("num_scale", ctypes.c_int64),
        ("num_embeds", ctypes.c_int64),
        ("dtype", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


class DAError(RuntimeError):
    def __init__(self, status: int, func: str, detail: str):
        self.status = status
        super().__init__(f"{func} failed with status {status}: {detail}")


_lib = None


def load() -> ctypes.CDLL:
    """Load libdeformagg.so; raises if it is missing (build it first)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m view_deformable_feature_amd.build` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32p = ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32)
    prob = ctypes.POINTER(DAProblem)
    lib.da_forward.argtypes = [prob, vp, i32p, i32p, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.da_forward.restype = ctypes.c_int
    lib.da_forward_workspace_size.argtypes = [prob, ctypes.POINTER(ctypes.c_size_t)]
    lib.da_forward_workspace_size.restype = ctypes.c_int
    for name in ("da_backward", "da_backward_accumulate"):
        f = getattr(lib, name)
        f.argtypes = [prob, vp, i32p, i32p, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        f.restype = ctypes.c_int
    for name in ("da_backward_atomic", "da_backward_noalloc"):
        f = getattr(lib, name)
        f.argtypes = [prob, vp, i32p, i32p, vp, vp, vp, vp, vp, vp, vp]
        f.restype = ctypes.c_int
    lib.da_backward_workspace_size.argtypes = [prob, ctypes.POINTER(ctypes.c_size_t)]
    lib.da_backward_workspace_size.restype = ctypes.c_int
    pprob = ctypes.POINTER(DAPackProblem)
    vpp = ctypes.POINTER(ctypes.c_void_p)
    lib.da_pack_layout.argtypes = [pprob, i32p, i32p, i32p, ctypes.POINTER(ctypes.c_int64)]
    lib.da_pack_layout.restype = ctypes.c_int
    lib.da_pack_levels.argtypes = [pprob, i32p, vpp, vp, vp]
    lib.da_pack_levels.restype = ctypes.c_int
    lib.da_unpack_levels.argtypes = [pprob, i32p, vp, vpp, vp]
    lib.da_unpack_levels.restype = ctypes.c_int
    dprob = ctypes.POINTER(DCNProblem)
    i64p, szp = ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_size_t)
    lib.dcn_out_size.argtypes = [dprob, i64p, i64p]
    lib.dcn_forward.argtypes = [dprob, vp, vp, vp, vp]
    lib.dcn_backward_workspace_size.argtypes = [dprob, szp]
    lib.dcn_backward.argtypes = [dprob, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    for name in ("dcn_out_size", "dcn_forward", "dcn_backward_workspace_size", "dcn_backward"):
        getattr(lib, name).restype = ctypes.c_int
    lib.da_status_string.argtypes = [ctypes.c_int]
    lib.da_status_string.restype = ctypes.c_char_p
    lib.da_last_error.argtypes = []
    lib.da_last_error.restype = ctypes.c_char_p
    lib.da_version.argtypes = []
    lib.da_version.restype = ctypes.c_int32
    _lib = lib
    return lib


def check(status: int, func: str) -> None:
    if status != DA_OK:
        lib = load()
        raise DAError(status, func, lib.da_last_error().decode(errors="replace"))


def declared_functions() -> List[str]:
    """Names of the functions the public headers (include/*.h) declare."""
    names = []
    for path in HEADER_PATHS:
        with open(path) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"\b((?:da|dcn)_[a-z_]+)\s*\(", text)
    return names
