"""fp64 CPU oracle for deformable aggregation (ctypes over ``oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the smoke check and by
the CPU-baseline leg of the benchmark.  The product library never imports,
links or calls anything here, and this package imports nothing from it.

The arithmetic lives in ``oracle.c`` (deformable aggregation) and
``dcn_oracle.c`` (deformable convolution); their headers state the definitions
they follow (the Sparse4D deformable_aggregation walkthrough,
mhpn.cn/news/1081857, sections 3.1, 3.2, 4.1 and 5.1; the DCNv4 paper notes,
docsaid.org, "Defining the problem") and the readings taken where the pages are
silent.  This file only marshals numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRCS = [os.path.join(_HERE, "oracle.c"), os.path.join(_HERE, "dcn_oracle.c")]
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

__all__ = ["build", "forward", "forward_parallel", "backward", "backward_anchors", "grad_feat_rows",
           "pack_levels", "unpack_levels", "dcn_out_size", "dcn_forward", "dcn_backward"]


def build(force: bool = True) -> str:
    """Compile the oracle sources into ``liboracle.so`` with gcc (no fast-math, no
    contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
                               "-fopenmp", "-fPIC", "-shared", *_SRCS, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or any(os.path.getmtime(_LIB) < os.path.getmtime(f)
                                           for f in _SRCS):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        i64, i32p, vp = ctypes.c_int64, ctypes.POINTER(ctypes.c_int32), ctypes.c_void_p
        prob = [i64] * 8 + [vp, ctypes.c_int, vp, vp, vp, vp]
        lib.oracle_forward.argtypes = prob + [vp, i64, vp]
        lib.oracle_forward_parallel.argtypes = prob + [ctypes.c_int, vp, vp]
        lib.oracle_backward.argtypes = prob + [vp, vp, vp, vp]
        lib.oracle_backward_anchors.argtypes = prob + [vp, vp, i64, vp, vp]
        lib.oracle_grad_feat_rows.argtypes = prob + [vp, vp, i64, vp]
        dcn = [i64] * 13
        lib.oracle_dcn_forward.argtypes = dcn + [vp, vp, vp]
        lib.oracle_dcn_backward.argtypes = dcn + [vp, vp, vp, vp, vp]
        lib.oracle_dcn_out_size.argtypes = dcn + [vp, vp]
        for f in (lib.oracle_forward, lib.oracle_forward_parallel, lib.oracle_backward, lib.oracle_backward_anchors,
                  lib.oracle_grad_feat_rows, lib.oracle_dcn_forward, lib.oracle_dcn_backward,
                  lib.oracle_dcn_out_size):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _problem(feat, spatial_shape, scale_start_index, loc, weights):
    """Validate dtypes/contiguity and derive the sizes; returns (args, keepalive, dims)."""
    spatial_shape = np.ascontiguousarray(spatial_shape, dtype=np.int32)
    scale_start_index = np.ascontiguousarray(scale_start_index, dtype=np.int32)
    K, S = scale_start_index.shape
    if feat.dtype == np.float16:
        feat = feat.astype(np.float32)          # exact: every binary16 value is a binary32 value
    if feat.dtype == np.uint16:
        is_bf16 = 1
    elif feat.dtype == np.float32:
        is_bf16 = 0
    else:
        raise TypeError("feat must be float32, float16 or uint16 bf16 bit patterns")
    feat = np.ascontiguousarray(feat)
    loc = np.ascontiguousarray(loc, dtype=np.float32)
    weights = np.ascontiguousarray(weights, dtype=np.float32)
    bs, num_feat, C = feat.shape
    A, P = loc.shape[1], loc.shape[2]
    G = weights.shape[-1]
    if loc.shape != (bs, A, P, K, 2) or weights.shape != (bs, A, P, K, S, G):
        raise ValueError("inconsistent shapes")
    dims = dict(bs=bs, num_feat=num_feat, C=C, A=A, P=P, K=K, S=S, G=G)
    args = [bs, num_feat, C, A, P, K, S, G, _ptr(feat), is_bf16, _ptr(spatial_shape),
            _ptr(scale_start_index), _ptr(loc), _ptr(weights)]
    return args, (feat, spatial_shape, scale_start_index, loc, weights), dims


def forward(feat, spatial_shape, scale_start_index, loc, weights,
            anchor_ids: Optional[Sequence[int]] = None) -> np.ndarray:
    """out [bs, A, C] (or [len(anchor_ids), C] for flat ids b*A + a), fp64."""
    args, keep, d = _problem(feat, spatial_shape, scale_start_index, loc, weights)
    if anchor_ids is None:
        out = np.empty((d["bs"], d["A"], d["C"]), dtype=np.float64)
        rc = _load().oracle_forward(*args, None, 0, _ptr(out))
    else:
        ids = np.ascontiguousarray(anchor_ids, dtype=np.int64)
        out = np.empty((ids.size, d["C"]), dtype=np.float64)
        rc = _load().oracle_forward(*args, _ptr(ids), ids.size, _ptr(out))
    if rc:
        raise ValueError(f"oracle_forward rejected the problem (rc={rc})")
    return out


def forward_parallel(feat, spatial_shape, scale_start_index, loc, weights,
                     threads: Optional[int] = None) -> Tuple[np.ndarray, int]:
    """(out [bs, A, C] fp64, threads used): the forward spread over OpenMP threads by
    anchor (all host cores by default); equal to forward() bit for bit."""
    args, keep, d = _problem(feat, spatial_shape, scale_start_index, loc, weights)
    n = int(threads or os.cpu_count() or 1)
    out = np.empty((d["bs"], d["A"], d["C"]), dtype=np.float64)
    used = ctypes.c_int(0)
    rc = _load().oracle_forward_parallel(*args, n, _ptr(out), ctypes.addressof(used))
    if rc:
        raise ValueError(f"oracle_forward_parallel rejected the problem (rc={rc})")
    return out, int(used.value)


def backward(feat, spatial_shape, scale_start_index, loc, weights, grad_out,
             need_feat: bool = True) -> Tuple[Optional[np.ndarray], np.ndarray, np.ndarray]:
    """(grad_feat [bs,num_feat,C] or None, grad_loc [bs,A,P,K,2], grad_weights [bs,A,P,K,S,G])."""
    args, keep, d = _problem(feat, spatial_shape, scale_start_index, loc, weights)
    if grad_out.dtype == np.uint16:
        raise TypeError("pass a bfloat16 grad_out as its float32 values")
    grad_out = np.ascontiguousarray(grad_out, dtype=np.float32)
    if grad_out.shape != (d["bs"], d["A"], d["C"]):
        raise ValueError("grad_out shape")
    gf = np.empty((d["bs"], d["num_feat"], d["C"]), dtype=np.float64) if need_feat else None
    gl = np.empty((d["bs"], d["A"], d["P"], d["K"], 2), dtype=np.float64)
    gw = np.empty((d["bs"], d["A"], d["P"], d["K"], d["S"], d["G"]), dtype=np.float64)
    rc = _load().oracle_backward(*args, _ptr(grad_out), _ptr(gf), _ptr(gl), _ptr(gw))
    if rc:
        raise ValueError(f"oracle_backward rejected the problem (rc={rc})")
    return gf, gl, gw


def backward_anchors(feat, spatial_shape, scale_start_index, loc, weights, grad_out,
                     anchor_ids: Sequence[int]) -> Tuple[np.ndarray, np.ndarray]:
    """grad_loc [n,P,K,2] and grad_weights [n,P,K,S,G] of flat anchors b*A + a."""
    args, keep, d = _problem(feat, spatial_shape, scale_start_index, loc, weights)
    grad_out = np.ascontiguousarray(grad_out, dtype=np.float32)
    ids = np.ascontiguousarray(anchor_ids, dtype=np.int64)
    gl = np.empty((ids.size, d["P"], d["K"], 2), dtype=np.float64)
    gw = np.empty((ids.size, d["P"], d["K"], d["S"], d["G"]), dtype=np.float64)
    rc = _load().oracle_backward_anchors(*args, _ptr(grad_out), _ptr(ids), ids.size,
                                         _ptr(gl), _ptr(gw))
    if rc:
        raise ValueError(f"oracle_backward_anchors rejected the problem (rc={rc})")
    return gl, gw


def grad_feat_rows(feat, spatial_shape, scale_start_index, loc, weights, grad_out,
                   rows: Sequence[int]) -> np.ndarray:
    """grad_feat of distinct flat rows b*num_feat + r: [n, C] fp64."""
    args, keep, d = _problem(feat, spatial_shape, scale_start_index, loc, weights)
    grad_out = np.ascontiguousarray(grad_out, dtype=np.float32)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.empty((rows.size, d["C"]), dtype=np.float64)
    rc = _load().oracle_grad_feat_rows(*args, _ptr(grad_out), _ptr(rows), rows.size, _ptr(out))
    if rc:
        raise ValueError(f"oracle_grad_feat_rows rejected the problem (rc={rc})")
    return out


def run_inputs(inp: Dict[str, np.ndarray], backward_too: bool = True):
    """Convenience: forward (and backward) of a ``make_inputs`` dict."""
    keys = ("feat", "spatial_shape", "scale_start_index", "loc", "weights")
    out = forward(*(inp[k] for k in keys))
    if not backward_too:
        return out
    return (out,) + backward(*(inp[k] for k in keys), inp["grad_out"])


# ---------------------------------------------------------------------------------------
# level packing (section 6: feature_maps_format), written out with numpy
# ---------------------------------------------------------------------------------------
# Layout (section 3.1 and the reading taken where section 6 is garbled): each
# (camera k, scale s) level is stored HWC -- pixel (i, j) of the level is row
# i*W + j of its block, C channels per row -- and the blocks follow camera by
# camera, scales in order inside a camera.  Pure rearrangement, no arithmetic.

def pack_levels(maps: Sequence[np.ndarray]):
    """maps[s]: [B, N, C, H_s, W_s] -> (packed [B, num_feat, C], spatial_shape [N, S, 2]
    int32, scale_start_index [N, S] int32)."""
    B, N, C = maps[0].shape[:3]
    S = len(maps)
    blocks, shape, start, row = [], np.zeros((N, S, 2), np.int32), np.zeros((N, S), np.int32), 0
    for k in range(N):
        for s, m in enumerate(maps):
            H, W = m.shape[3], m.shape[4]
            # [B, C, H, W] -> [B, H, W, C] -> [B, H*W, C]
            blocks.append(np.transpose(m[:, k], (0, 2, 3, 1)).reshape(B, H * W, C))
            shape[k, s] = (H, W)
            start[k, s] = row
            row += H * W
    return np.ascontiguousarray(np.concatenate(blocks, axis=1)), shape, start


def unpack_levels(packed: np.ndarray, scale_hw: Sequence[Tuple[int, int]], num_cams: int):
    """The inverse of pack_levels: packed [B, num_feat, C] -> list of [B, N, C, H_s, W_s]."""
    B, _, C = packed.shape
    maps = [np.empty((B, num_cams, C, h, w), packed.dtype) for h, w in scale_hw]
    row = 0
    for k in range(num_cams):
        for s, (h, w) in enumerate(scale_hw):
            block = packed[:, row:row + h * w, :].reshape(B, h, w, C)
            maps[s][:, k] = np.transpose(block, (0, 3, 1, 2))
            row += h * w
    return maps


# ---------------------------------------------------------------------------------------
# deformable convolution (dcn_oracle.c)
# ---------------------------------------------------------------------------------------

def _pair(v) -> Tuple[int, int]:
    return (int(v), int(v)) if np.isscalar(v) else (int(v[0]), int(v[1]))


def _dcn_input(x: np.ndarray) -> np.ndarray:
    """float32 values of the input (binary16 converts exactly); bfloat16 comes as
    its uint16 bit patterns."""
    if x.dtype == np.uint16:
        return (np.ascontiguousarray(x).astype(np.uint32) << np.uint32(16)).view(np.float32)
    if x.dtype not in (np.float32, np.float16):
        raise TypeError("input must be float32, float16 or uint16 bfloat16 bit patterns")
    return np.ascontiguousarray(x, dtype=np.float32)


def _dcn_args(x, groups, kernel, stride, pad, dilation):
    N, H, W, C = x.shape
    kh, kw = _pair(kernel)
    sh, sw = _pair(stride)
    ph, pw = _pair(pad)
    dh, dw = _pair(dilation)
    return [N, H, W, C, int(groups), kh, kw, sh, sw, ph, pw, dh, dw]


def dcn_out_size(H, W, kernel=3, stride=1, pad=1, dilation=1) -> Tuple[int, int]:
    args = [1, H, W, 1, 1, *_pair(kernel), *_pair(stride), *_pair(pad), *_pair(dilation)]
    ho, wo = ctypes.c_int64(0), ctypes.c_int64(0)
    rc = _load().oracle_dcn_out_size(*args, ctypes.byref(ho), ctypes.byref(wo))
    if rc:
        raise ValueError(f"oracle_dcn_out_size rejected the problem (rc={rc})")
    return ho.value, wo.value


def dcn_forward(x, offset_mask, groups, kernel=3, stride=1, pad=1, dilation=1) -> np.ndarray:
    """x [N, H, W, C], offset_mask [N, Ho, Wo, G, 3K] float32 -> out [N, Ho, Wo, C] fp64."""
    xf = _dcn_input(x)
    args = _dcn_args(xf, groups, kernel, stride, pad, dilation)
    ho, wo = dcn_out_size(args[1], args[2], kernel, stride, pad, dilation)
    K = args[5] * args[6]
    om = np.ascontiguousarray(offset_mask, dtype=np.float32)
    if om.shape != (args[0], ho, wo, args[4], 3 * K):
        raise ValueError(f"offset_mask shape {om.shape}")
    out = np.empty((args[0], ho, wo, args[3]), dtype=np.float64)
    rc = _load().oracle_dcn_forward(*args, _ptr(xf), _ptr(om), _ptr(out))
    if rc:
        raise ValueError(f"oracle_dcn_forward rejected the problem (rc={rc})")
    return out


def dcn_backward(x, offset_mask, grad_out, groups, kernel=3, stride=1, pad=1, dilation=1):
    """(grad_input [N, H, W, C], grad_offset_mask [N, Ho, Wo, G, 3K]), fp64."""
    xf = _dcn_input(x)
    args = _dcn_args(xf, groups, kernel, stride, pad, dilation)
    ho, wo = dcn_out_size(args[1], args[2], kernel, stride, pad, dilation)
    K = args[5] * args[6]
    om = np.ascontiguousarray(offset_mask, dtype=np.float32)
    if om.shape != (args[0], ho, wo, args[4], 3 * K):
        raise ValueError(f"offset_mask shape {om.shape}")
    if np.asarray(grad_out).dtype == np.uint16:
        raise TypeError("pass a bfloat16 grad_out as its float32 values")
    go = np.ascontiguousarray(grad_out, dtype=np.float32)
    if go.shape != (args[0], ho, wo, args[3]):
        raise ValueError(f"grad_out shape {go.shape}")
    gi = np.empty(xf.shape, dtype=np.float64)
    gom = np.empty(om.shape, dtype=np.float64)
    rc = _load().oracle_dcn_backward(*args, _ptr(xf), _ptr(om), _ptr(go), _ptr(gi), _ptr(gom))
    if rc:
        raise ValueError(f"oracle_dcn_backward rejected the problem (rc={rc})")
    return gi, gom
