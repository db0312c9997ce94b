"""PyTorch-facing binding of libdeformagg.

Same names as the C ABI (``da_forward``, ``da_backward``,
``da_backward_accumulate``, ``da_backward_atomic``) plus the autograd wrapper
``DeformableAggregationFunction`` whose ``forward(ctx, mc_ms_feat,
spatial_shape, scale_start_index, sampling_location, weights)`` follows the
signature shown in section 6 of the Sparse4D deformable_aggregation
walkthrough (mhpn.cn/news/1081857).

This module only checks tensor metadata and passes pointers: every step of
the computation runs in the HIP kernels of libdeformagg.  torch supplies
device memory and the current stream.
"""
from __future__ import annotations

import ctypes
from collections import OrderedDict
from typing import Optional, Sequence, Tuple, Union

import numpy as np
import torch

from . import _lib

__all__ = ["da_forward", "da_backward", "da_backward_accumulate", "da_backward_atomic",
           "workspace_size", "forward_workspace_size", "DeformableAggregationFunction",
           "deformable_aggregation", "problem_of"]

IntTable = Union[torch.Tensor, np.ndarray, Sequence]

# torch dtype -> da_dtype, for mc_ms_feat and for out / grad_out
_DTYPES = {torch.float32: _lib.DA_F32, torch.bfloat16: _lib.DA_BF16, torch.float16: _lib.DA_F16}
_FLOATS = tuple(_DTYPES)


# Host copies of device-resident level tables, keyed on the tensor's identity and
# torch's version counter (bumped by every in-place update through torch).  Each
# entry holds a reference to its tensor, so that its memory -- and so the key --
# cannot be reused while cached.  A table that only kernels outside torch rewrite
# in place would be served stale: level tables are constants in practice.
_TABLE_CACHE: "OrderedDict[tuple, tuple]" = OrderedDict()
_TABLE_CACHE_SIZE = 32


def _host_i32(x: IntTable) -> np.ndarray:
    """Level tables are read on the host.  A CPU tensor or array is converted; a device
    tensor is copied to the host (one blocking copy) the first time it is seen, and
    later calls with the same unchanged tensor reuse that copy without synchronising."""
    if isinstance(x, torch.Tensor):
        if x.device.type == "cpu":
            x = x.detach().numpy()
        else:
            key = (id(x), x.data_ptr(), x._version, tuple(x.shape), x.dtype, str(x.device))
            hit = _TABLE_CACHE.get(key)
            if hit is not None and hit[0] is x:
                _TABLE_CACHE.move_to_end(key)
                return hit[1]
            host = np.ascontiguousarray(x.detach().to("cpu").numpy(), dtype=np.int32)
            host.setflags(write=False)
            _TABLE_CACHE[key] = (x, host)
            while len(_TABLE_CACHE) > _TABLE_CACHE_SIZE:
                _TABLE_CACHE.popitem(last=False)
            return host
    return np.ascontiguousarray(np.asarray(x), dtype=np.int32)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t: torch.Tensor, name: str, dtype, device, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU (got {t.device}); there is no CPU path")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _flags(slices: Optional[bool], regather: Optional[bool] = None,
           deterministic: bool = False) -> int:
    """slices: None lets the library choose level slices, True / False force them on /
    off.  regather: None lets the library choose the backward form; True takes the
    per-anchor form that gathers the corner rows again, False the row-ordered form
    (where the lane layout allows it)."""
    f = 0
    if slices is not None:
        f |= _lib.DA_FLAG_SLICES_ALWAYS if slices else _lib.DA_FLAG_SLICES_NEVER
    if regather is not None:
        f |= _lib.DA_FLAG_BWD_REGATHER if regather else _lib.DA_FLAG_BWD_ROW_ORDER
    if deterministic:
        f |= _lib.DA_FLAG_DETERMINISTIC
    return f


def problem_of(mc_ms_feat: torch.Tensor, spatial_shape: np.ndarray,
               sampling_location: torch.Tensor, weights: torch.Tensor,
               slices: Optional[bool] = None, regather: Optional[bool] = None,
               deterministic: bool = False,
               out_dtype: torch.dtype = torch.float32) -> _lib.DAProblem:
    if mc_ms_feat.dim() != 3:
        raise ValueError("mc_ms_feat must be [bs, num_feat, C]")
    if sampling_location.dim() != 5 or sampling_location.shape[-1] != 2:
        raise ValueError("sampling_location must be [bs, A, P, K, 2]")
    if weights.dim() != 6:
        raise ValueError("weights must be [bs, A, P, K, S, G]")
    if spatial_shape.ndim != 3 or spatial_shape.shape[-1] != 2:
        raise ValueError("spatial_shape must be [num_cams, num_scale, 2]")
    bs, num_feat, C = mc_ms_feat.shape
    _, A, P, K, _ = sampling_location.shape
    S, G = weights.shape[4], weights.shape[5]
    if spatial_shape.shape[:2] != (K, S):
        raise ValueError(f"spatial_shape is {spatial_shape.shape}, expected ({K}, {S}, 2)")
    if mc_ms_feat.dtype not in _DTYPES or out_dtype not in _DTYPES:
        raise TypeError(f"feature / output dtypes must be among {_FLOATS}")
    return _lib.DAProblem(bs, num_feat, C, A, P, K, S, G, _DTYPES[mc_ms_feat.dtype],
                          _flags(slices, regather, deterministic), _DTYPES[out_dtype], 0)


def _prepare(mc_ms_feat, spatial_shape, scale_start_index, sampling_location, weights,
             slices=None, regather=None, deterministic=False, out_dtype=torch.float32):
    shape = _host_i32(spatial_shape)
    start = _host_i32(scale_start_index)
    dev = mc_ms_feat.device
    _need(mc_ms_feat, "mc_ms_feat", _FLOATS, dev)
    _need(sampling_location, "sampling_location", torch.float32, dev)
    _need(weights, "weights", torch.float32, dev)
    prob = problem_of(mc_ms_feat, shape, sampling_location, weights, slices, regather,
                      deterministic, out_dtype)
    bs, A, P, K = (sampling_location.shape[i] for i in range(4))
    if tuple(weights.shape[:4]) != (bs, A, P, K) or mc_ms_feat.shape[0] != bs:
        raise ValueError("batch / anchor / point / camera sizes disagree between inputs")
    if start.shape != shape.shape[:2]:
        raise ValueError(f"scale_start_index is {start.shape}, expected {shape.shape[:2]}")
    return prob, shape, start


def _i32p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _stream(device: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _workspace(lib, size_fn: str, prob, dev, workspace):
    """The caller's workspace, checked, or a new one from torch's caching allocator
    (no device allocation on the steady path); None when none is needed."""
    n = ctypes.c_size_t(0)
    _lib.check(getattr(lib, size_fn)(ctypes.byref(prob), ctypes.byref(n)), size_fn)
    if workspace is None and n.value:
        workspace = torch.empty(int(n.value), device=dev, dtype=torch.uint8)
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, dev)
        if workspace.numel() < n.value:
            raise ValueError(f"workspace has {workspace.numel()} bytes, {n.value} needed")
    return workspace


def da_forward(mc_ms_feat: torch.Tensor, spatial_shape: IntTable, scale_start_index: IntTable,
               sampling_location: torch.Tensor, weights: torch.Tensor,
               out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
               slices: Optional[bool] = None,
               out_dtype: Optional[torch.dtype] = None) -> torch.Tensor:
    """out[bs, A, C] on the current stream of mc_ms_feat's device.

    The type of out is that of a given ``out`` tensor, else ``out_dtype`` (float32 by
    default; bfloat16 / float16 round the binary32 sums once, to nearest even).

    slices=None lets the library choose level slices (given a workspace, allocated
    here when not passed), True forces them, False runs one workgroup per anchor."""
    lib = _lib.load()
    if out is not None and out_dtype is not None and out.dtype != out_dtype:
        raise TypeError(f"out has dtype {out.dtype}, out_dtype is {out_dtype}")
    odt = out.dtype if out is not None else (out_dtype or torch.float32)
    prob, shape, start = _prepare(mc_ms_feat, spatial_shape, scale_start_index,
                                  sampling_location, weights, slices, out_dtype=odt)
    dev = mc_ms_feat.device
    if out is None:
        out = torch.empty((prob.bs, prob.num_anchors, prob.num_embeds), device=dev, dtype=odt)
    _need(out, "out", _FLOATS, dev, (prob.bs, prob.num_anchors, prob.num_embeds))
    workspace = _workspace(lib, "da_forward_workspace_size", prob, dev, workspace)
    with torch.cuda.device(dev):
        st = lib.da_forward(ctypes.byref(prob), _ptr(mc_ms_feat), _i32p(shape), _i32p(start),
                            _ptr(sampling_location), _ptr(weights), _ptr(out), _ptr(workspace),
                            0 if workspace is None else workspace.numel(), _stream(dev))
    _lib.check(st, "da_forward")
    return out


def forward_workspace_size(mc_ms_feat, spatial_shape, sampling_location, weights,
                           slices: Optional[bool] = None) -> int:
    """Bytes of workspace that let da_forward use level slices for these shapes."""
    lib = _lib.load()
    prob = problem_of(mc_ms_feat, _host_i32(spatial_shape), sampling_location, weights, slices)
    n = ctypes.c_size_t(0)
    _lib.check(lib.da_forward_workspace_size(ctypes.byref(prob), ctypes.byref(n)),
               "da_forward_workspace_size")
    return int(n.value)


def workspace_size(mc_ms_feat, spatial_shape, sampling_location, weights,
                   regather: Optional[bool] = None, deterministic: bool = False,
                   grad_out_dtype: torch.dtype = torch.float32) -> int:
    """Bytes of workspace da_backward / da_backward_accumulate need for these shapes
    (and a grad_out of grad_out_dtype)."""
    lib = _lib.load()
    prob = problem_of(mc_ms_feat, _host_i32(spatial_shape), sampling_location, weights,
                      regather=regather, deterministic=deterministic, out_dtype=grad_out_dtype)
    n = ctypes.c_size_t(0)
    _lib.check(lib.da_backward_workspace_size(ctypes.byref(prob), ctypes.byref(n)),
               "da_backward_workspace_size")
    return int(n.value)


def _backward(func: str, mc_ms_feat, spatial_shape, scale_start_index, sampling_location,
              weights, grad_out, grad_feat=None, grad_loc=None, grad_weights=None,
              workspace=None, slices=None, regather=None, deterministic=False):
    lib = _lib.load()
    if not isinstance(grad_out, torch.Tensor) or grad_out.dtype not in _DTYPES:
        raise TypeError(f"grad_out must be a tensor of one of {_FLOATS}")
    prob, shape, start = _prepare(mc_ms_feat, spatial_shape, scale_start_index,
                                  sampling_location, weights, slices, regather, deterministic,
                                  grad_out.dtype)
    dev = mc_ms_feat.device
    _need(grad_out, "grad_out", _FLOATS, dev, (prob.bs, prob.num_anchors, prob.num_embeds))
    if grad_feat is None:
        if func == "da_backward_accumulate":
            raise ValueError("da_backward_accumulate needs an existing grad_feat")
        grad_feat = torch.empty(tuple(mc_ms_feat.shape), device=dev, dtype=torch.float32)
    if grad_loc is None:
        grad_loc = torch.empty(tuple(sampling_location.shape), device=dev, dtype=torch.float32)
    if grad_weights is None:
        grad_weights = torch.empty(tuple(weights.shape), device=dev, dtype=torch.float32)
    _need(grad_feat, "grad_feat", torch.float32, dev, tuple(mc_ms_feat.shape))
    _need(grad_loc, "grad_loc", torch.float32, dev, tuple(sampling_location.shape))
    _need(grad_weights, "grad_weights", torch.float32, dev, tuple(weights.shape))
    with torch.cuda.device(dev):
        common = (ctypes.byref(prob), _ptr(mc_ms_feat), _i32p(shape), _i32p(start),
                  _ptr(sampling_location), _ptr(weights), _ptr(grad_out), _ptr(grad_feat),
                  _ptr(grad_loc), _ptr(grad_weights))
        if func == "da_backward_atomic":
            st = lib.da_backward_atomic(*common, _stream(dev))
        else:
            workspace = _workspace(lib, "da_backward_workspace_size", prob, dev, workspace)
            st = getattr(lib, func)(*common, _ptr(workspace),
                                    0 if workspace is None else workspace.numel(), _stream(dev))
    _lib.check(st, func)
    return grad_feat, grad_loc, grad_weights


def da_backward(mc_ms_feat, spatial_shape, scale_start_index, sampling_location, weights,
                grad_out, grad_feat=None, grad_loc=None, grad_weights=None, workspace=None,
                slices=None, regather=None, deterministic=False
                ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """(grad_feat [bs,num_feat,C] f32, grad_loc [bs,A,P,K,2], grad_weights [bs,A,P,K,S,G]).

    grad_out may be float32, bfloat16 or float16 (the type the forward wrote out in).

    deterministic=True: grad_feat bit for bit independent of run, backward form and
    level slices (64-bit fixed-point sums; needs finite grad_out and weights)."""
    return _backward("da_backward", mc_ms_feat, spatial_shape, scale_start_index,
                     sampling_location, weights, grad_out, grad_feat, grad_loc, grad_weights,
                     workspace, slices, regather, deterministic)


def da_backward_accumulate(mc_ms_feat, spatial_shape, scale_start_index, sampling_location,
                           weights, grad_out, grad_feat, grad_loc=None, grad_weights=None,
                           workspace=None, slices=None, regather=None, deterministic=False):
    """As da_backward, adding the feature gradient into the existing ``grad_feat``."""
    return _backward("da_backward_accumulate", mc_ms_feat, spatial_shape, scale_start_index,
                     sampling_location, weights, grad_out, grad_feat, grad_loc, grad_weights,
                     workspace, slices, regather, deterministic)


def da_backward_atomic(mc_ms_feat, spatial_shape, scale_start_index, sampling_location,
                       weights, grad_out, grad_feat=None, grad_loc=None, grad_weights=None):
    """As da_backward, with the feature gradient scattered by binary32 atomics (no workspace)."""
    return _backward("da_backward_atomic", mc_ms_feat, spatial_shape, scale_start_index,
                     sampling_location, weights, grad_out, grad_feat, grad_loc, grad_weights)


class DeformableAggregationFunction(torch.autograd.Function):
    """Autograd wrapper: gradients for mc_ms_feat, sampling_location and weights.

    The feature gradient is float32 (for 16-bit features it is cast back to the
    feature type for autograd; use ``da_backward`` directly to keep the float32
    values).  ``out_dtype`` (after the page's five arguments) picks the output type.
    """

    @staticmethod
    def forward(ctx, mc_ms_feat, spatial_shape, scale_start_index, sampling_location, weights,
                out_dtype=None):
        shape = _host_i32(spatial_shape)
        start = _host_i32(scale_start_index)
        mc_ms_feat = mc_ms_feat.contiguous()
        sampling_location = sampling_location.contiguous().float()
        weights = weights.contiguous().float()
        out = da_forward(mc_ms_feat, shape, start, sampling_location, weights,
                         out_dtype=out_dtype)
        ctx.save_for_backward(mc_ms_feat, sampling_location, weights)
        ctx.tables = (shape, start)
        return out

    @staticmethod
    def backward(ctx, grad_out):
        mc_ms_feat, sampling_location, weights = ctx.saved_tensors
        shape, start = ctx.tables
        if grad_out.dtype not in _DTYPES:
            grad_out = grad_out.float()
        gf, gl, gw = da_backward(mc_ms_feat, shape, start, sampling_location, weights,
                                 grad_out.contiguous())
        if mc_ms_feat.dtype != torch.float32:
            gf = gf.to(mc_ms_feat.dtype)
        return gf, None, None, gl, gw, None


def deformable_aggregation(mc_ms_feat, spatial_shape, scale_start_index, sampling_location,
                           weights, out_dtype=None):
    return DeformableAggregationFunction.apply(mc_ms_feat, spatial_shape, scale_start_index,
                                               sampling_location, weights, out_dtype)
