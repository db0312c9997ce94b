"""Binding of the level-packing entry points (da_pack_layout, da_pack_levels,
da_unpack_levels) and ``feature_maps_format`` built on them.

Section 6 of the Sparse4D deformable_aggregation walkthrough
(mhpn.cn/news/1081857) names ``feature_maps_format(feature_maps, inverse)``:
per-scale camera maps ``[B, N, C, H_s, W_s]`` to ``[mc_ms_feat, spatial_shape,
scale_start_index]`` and back.  The packed layout is the one the aggregation
reads (section 3.1, HWC per level; levels camera-major, scales in order).
Every step runs in the HIP kernels of libdeformagg; this module checks tensor
metadata and passes pointers.
"""
from __future__ import annotations

import ctypes
from typing import List, Optional, Sequence, Tuple

import numpy as np
import torch

from . import _lib
from .api import _need, _stream

__all__ = ["pack_layout", "da_pack_levels", "da_unpack_levels", "pack_levels",
           "PackLevelsFunction", "feature_maps_format"]


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return _lib.DA_F32
    if dt == torch.bfloat16:
        return _lib.DA_BF16
    if dt == torch.float16:
        return _lib.DA_F16
    raise TypeError(f"packing supports float32, bfloat16 and float16 maps, got {dt}")


def _problem(bs, num_cams, num_scale, C, dtype) -> _lib.DAPackProblem:
    return _lib.DAPackProblem(bs, num_cams, num_scale, C, _dtype_code(dtype), 0)


def _scale_hw(shapes: Sequence[Tuple[int, int]]) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(shapes, dtype=np.int32).reshape(-1, 2))


def _i32p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def pack_layout(scale_hw, num_cams: int, C: int = 1, dtype=torch.float32):
    """(spatial_shape [N, S, 2], scale_start_index [N, S], num_feat) for scales of
    (H, W) = scale_hw[s], computed by the library (host only)."""
    lib = _lib.load()
    hw = _scale_hw(scale_hw)
    prob = _problem(1, num_cams, hw.shape[0], C, dtype)
    shape = np.zeros((num_cams, hw.shape[0], 2), np.int32)
    start = np.zeros((num_cams, hw.shape[0]), np.int32)
    nf = ctypes.c_int64(0)
    _lib.check(lib.da_pack_layout(ctypes.byref(prob), _i32p(hw), _i32p(shape), _i32p(start),
                                  ctypes.byref(nf)), "da_pack_layout")
    return shape, start, int(nf.value)


def _maps_meta(maps: Sequence[torch.Tensor]):
    if len(maps) == 0:
        raise ValueError("need at least one scale")
    B, N, C = maps[0].shape[:3]
    dev, dt = maps[0].device, maps[0].dtype
    for m in maps:
        if m.dim() != 5 or tuple(m.shape[:3]) != (B, N, C):
            raise ValueError("every map must be [B, N, C, H, W] with the same B, N, C")
        _need(m, "feature map", dt, dev)
    return B, N, C, dev, dt, [(int(m.shape[3]), int(m.shape[4])) for m in maps]


def da_pack_levels(maps: Sequence[torch.Tensor], out: Optional[torch.Tensor] = None
                   ) -> torch.Tensor:
    """packed [B, num_feat, C] from per-scale maps [B, N, C, H_s, W_s]."""
    lib = _lib.load()
    B, N, C, dev, dt, shapes = _maps_meta(maps)
    hw = _scale_hw(shapes)
    _, _, nf = pack_layout(shapes, N, C, dt)
    if out is None:
        out = torch.empty((B, nf, C), device=dev, dtype=dt)
    _need(out, "packed", dt, dev, (B, nf, C))
    ptrs = (ctypes.c_void_p * len(maps))(*[m.data_ptr() for m in maps])
    prob = _problem(B, N, len(maps), C, dt)
    with torch.cuda.device(dev):
        st = lib.da_pack_levels(ctypes.byref(prob), _i32p(hw), ptrs, ctypes.c_void_p(out.data_ptr()),
                                _stream(dev))
    _lib.check(st, "da_pack_levels")
    return out


def da_unpack_levels(packed: torch.Tensor, scale_hw, num_cams: int,
                     out: Optional[List[torch.Tensor]] = None) -> List[torch.Tensor]:
    """Per-scale maps [B, N, C, H_s, W_s] from packed [B, num_feat, C]."""
    lib = _lib.load()
    if packed.dim() != 3:
        raise ValueError("packed must be [B, num_feat, C]")
    B, nf, C = packed.shape
    dev, dt = packed.device, packed.dtype
    _need(packed, "packed", dt, dev)
    hw = _scale_hw(scale_hw)
    _, _, nf_expect = pack_layout(hw, num_cams, C, dt)
    if nf != nf_expect:
        raise ValueError(f"packed has {nf} rows, the levels need {nf_expect}")
    if out is None:
        out = [torch.empty((B, num_cams, C, int(h), int(w)), device=dev, dtype=dt) for h, w in hw]
    for m, (h, w) in zip(out, hw):
        _need(m, "feature map", dt, dev, (B, num_cams, C, int(h), int(w)))
    ptrs = (ctypes.c_void_p * len(out))(*[m.data_ptr() for m in out])
    prob = _problem(B, num_cams, hw.shape[0], C, dt)
    with torch.cuda.device(dev):
        st = lib.da_unpack_levels(ctypes.byref(prob), _i32p(hw), ctypes.c_void_p(packed.data_ptr()),
                                  ptrs, _stream(dev))
    _lib.check(st, "da_unpack_levels")
    return out


class PackLevelsFunction(torch.autograd.Function):
    """packed = pack(maps); the gradient of each map is the unpacked gradient."""

    @staticmethod
    def forward(ctx, *maps):
        maps = [m.contiguous() for m in maps]
        ctx.shapes = [(int(m.shape[3]), int(m.shape[4])) for m in maps]
        ctx.num_cams = int(maps[0].shape[1])
        return da_pack_levels(maps)

    @staticmethod
    def backward(ctx, grad_packed):
        return tuple(da_unpack_levels(grad_packed.contiguous(), ctx.shapes, ctx.num_cams))


def pack_levels(maps: Sequence[torch.Tensor]) -> torch.Tensor:
    return PackLevelsFunction.apply(*maps)


def feature_maps_format(feature_maps, inverse: bool = False):
    """inverse=False: list of [B, N, C, H_s, W_s] maps -> [mc_ms_feat, spatial_shape,
    scale_start_index] (the level table as int32 tensors on the maps' device).
    inverse=True: [mc_ms_feat, spatial_shape, scale_start_index] -> the list of maps."""
    if not inverse:
        maps = list(feature_maps)
        _, N, C, dev, dt, shapes = _maps_meta(maps)
        shape, start, _ = pack_layout(shapes, N, C, dt)
        return [pack_levels(maps), torch.from_numpy(shape).to(dev),
                torch.from_numpy(start).to(dev)]
    packed, spatial_shape, scale_start_index = feature_maps
    shape = spatial_shape.detach().cpu().numpy() if isinstance(spatial_shape, torch.Tensor) \
        else np.asarray(spatial_shape)
    start = scale_start_index.detach().cpu().numpy() if isinstance(scale_start_index, torch.Tensor) \
        else np.asarray(scale_start_index)
    N = shape.shape[0]
    if not (shape == shape[:1]).all():
        raise ValueError("inverse packing needs the same (H, W) per scale for every camera")
    exp_shape, exp_start, _ = pack_layout(shape[0], N, packed.shape[-1], packed.dtype)
    if not np.array_equal(exp_start, start):
        raise ValueError("scale_start_index is not the camera-major packed layout")
    return da_unpack_levels(packed, shape[0], N)
