"""PyTorch binding of the deformable convolution in libdeformagg (include/dcn.h).

The operator is the one the DCNv4 paper notes (docsaid.org, "DCNv4") define in
"Defining the problem": each group of C / G channels sums, over the taps of a
kernel grid, a modulation scalar times its input sampled bilinearly at the tap
plus a learned offset; DCNv4 leaves the scalars unbounded.  Tensors are
channel-last: input [N, H, W, C], offset_mask [N, Ho, Wo, G, 3K] ((dx, dy) per tap,
then the K scalars), out [N, Ho, Wo, C].

Only metadata checks and pointer passing happen here; every step runs in the HIP
kernels of libdeformagg.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Tuple, Union

import torch

from . import _lib
from .api import _DTYPES, _FLOATS, _need, _ptr, _stream

__all__ = ["dcn_out_size", "dcn_forward", "dcn_backward", "dcn_workspace_size",
           "DCNFunction", "deformable_conv"]

Pair = Union[int, Tuple[int, int]]


def _pair(v: Pair) -> Tuple[int, int]:
    return (int(v), int(v)) if isinstance(v, int) else (int(v[0]), int(v[1]))


def _problem(shape, groups, kernel, stride, pad, dilation, in_dtype, out_dtype) -> _lib.DCNProblem:
    N, H, W, C = shape
    (kh, kw), (sh, sw), (ph, pw), (dh, dw) = (_pair(kernel), _pair(stride), _pair(pad),
                                              _pair(dilation))
    if in_dtype not in _DTYPES or out_dtype not in _DTYPES:
        raise TypeError(f"input / output dtypes must be among {_FLOATS}")
    return _lib.DCNProblem(N, H, W, C, int(groups), kh, kw, sh, sw, ph, pw, dh, dw,
                           _DTYPES[in_dtype], _DTYPES[out_dtype], 0, 0)


def dcn_out_size(height: int, width: int, kernel: Pair = 3, stride: Pair = 1, pad: Pair = 1,
                 dilation: Pair = 1) -> Tuple[int, int]:
    lib = _lib.load()
    prob = _problem((1, height, width, 1), 1, kernel, stride, pad, dilation, torch.float32,
                    torch.float32)
    ho, wo = ctypes.c_int64(0), ctypes.c_int64(0)
    _lib.check(lib.dcn_out_size(ctypes.byref(prob), ctypes.byref(ho), ctypes.byref(wo)),
               "dcn_out_size")
    return int(ho.value), int(wo.value)


def _check_inputs(input, offset_mask, groups, kernel, stride, pad, dilation):
    if not isinstance(input, torch.Tensor) or input.dim() != 4:
        raise ValueError("input must be a [N, H, W, C] tensor")
    dev = input.device
    _need(input, "input", _FLOATS, dev)
    N, H, W, C = input.shape
    ho, wo = dcn_out_size(H, W, kernel, stride, pad, dilation)
    kh, kw = _pair(kernel)
    _need(offset_mask, "offset_mask", torch.float32, dev, (N, ho, wo, int(groups), 3 * kh * kw))
    return dev, (N, H, W, C), (ho, wo)


def dcn_forward(input: torch.Tensor, offset_mask: torch.Tensor, groups: int, kernel: Pair = 3,
                stride: Pair = 1, pad: Pair = 1, dilation: Pair = 1,
                out: Optional[torch.Tensor] = None,
                out_dtype: Optional[torch.dtype] = None) -> torch.Tensor:
    """out [N, Ho, Wo, C] (float32 unless ``out`` / ``out_dtype`` says otherwise; a
    16-bit out is the binary32 sum rounded once to nearest even)."""
    lib = _lib.load()
    dev, shape, (ho, wo) = _check_inputs(input, offset_mask, groups, kernel, stride, pad, dilation)
    odt = out.dtype if out is not None else (out_dtype or torch.float32)
    prob = _problem(shape, groups, kernel, stride, pad, dilation, input.dtype, odt)
    if out is None:
        out = torch.empty((shape[0], ho, wo, shape[3]), device=dev, dtype=odt)
    _need(out, "out", _FLOATS, dev, (shape[0], ho, wo, shape[3]))
    with torch.cuda.device(dev):
        st = lib.dcn_forward(ctypes.byref(prob), _ptr(input), _ptr(offset_mask), _ptr(out),
                             _stream(dev))
    _lib.check(st, "dcn_forward")
    return out


def dcn_workspace_size(input: torch.Tensor, groups: int, kernel: Pair = 3, stride: Pair = 1,
                       pad: Pair = 1, dilation: Pair = 1,
                       grad_out_dtype: torch.dtype = torch.float32) -> int:
    lib = _lib.load()
    prob = _problem(tuple(input.shape), groups, kernel, stride, pad, dilation, input.dtype,
                    grad_out_dtype)
    n = ctypes.c_size_t(0)
    _lib.check(lib.dcn_backward_workspace_size(ctypes.byref(prob), ctypes.byref(n)),
               "dcn_backward_workspace_size")
    return int(n.value)


def dcn_backward(input: torch.Tensor, offset_mask: torch.Tensor, grad_out: torch.Tensor,
                 groups: int, kernel: Pair = 3, stride: Pair = 1, pad: Pair = 1,
                 dilation: Pair = 1, grad_input: Optional[torch.Tensor] = None,
                 grad_offset_mask: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None
                 ) -> Tuple[torch.Tensor, torch.Tensor]:
    """(grad_input [N, H, W, C] float32, grad_offset_mask [N, Ho, Wo, G, 3K] float32)."""
    lib = _lib.load()
    dev, shape, (ho, wo) = _check_inputs(input, offset_mask, groups, kernel, stride, pad, dilation)
    if not isinstance(grad_out, torch.Tensor) or grad_out.dtype not in _DTYPES:
        raise TypeError(f"grad_out must be a tensor of one of {_FLOATS}")
    _need(grad_out, "grad_out", _FLOATS, dev, (shape[0], ho, wo, shape[3]))
    prob = _problem(shape, groups, kernel, stride, pad, dilation, input.dtype, grad_out.dtype)
    if grad_input is None:
        grad_input = torch.empty(shape, device=dev, dtype=torch.float32)
    if grad_offset_mask is None:
        grad_offset_mask = torch.empty(tuple(offset_mask.shape), device=dev, dtype=torch.float32)
    _need(grad_input, "grad_input", torch.float32, dev, shape)
    _need(grad_offset_mask, "grad_offset_mask", torch.float32, dev, tuple(offset_mask.shape))
    n = ctypes.c_size_t(0)
    _lib.check(lib.dcn_backward_workspace_size(ctypes.byref(prob), ctypes.byref(n)),
               "dcn_backward_workspace_size")
    if workspace is None and n.value:
        workspace = torch.empty(int(n.value), device=dev, dtype=torch.uint8)
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, dev)
        if workspace.numel() < n.value:
            raise ValueError(f"workspace has {workspace.numel()} bytes, {n.value} needed")
    with torch.cuda.device(dev):
        st = lib.dcn_backward(ctypes.byref(prob), _ptr(input), _ptr(offset_mask), _ptr(grad_out),
                              _ptr(grad_input), _ptr(grad_offset_mask), _ptr(workspace),
                              0 if workspace is None else workspace.numel(), _stream(dev))
    _lib.check(st, "dcn_backward")
    return grad_input, grad_offset_mask


class DCNFunction(torch.autograd.Function):
    """Autograd wrapper: gradients for input (cast to its type) and offset_mask."""

    @staticmethod
    def forward(ctx, input, offset_mask, groups, kernel=3, stride=1, pad=1, dilation=1,
                out_dtype=None):
        input = input.contiguous()
        offset_mask = offset_mask.contiguous().float()
        out = dcn_forward(input, offset_mask, groups, kernel, stride, pad, dilation,
                          out_dtype=out_dtype)
        ctx.save_for_backward(input, offset_mask)
        ctx.conf = (groups, kernel, stride, pad, dilation)
        return out

    @staticmethod
    def backward(ctx, grad_out):
        input, offset_mask = ctx.saved_tensors
        if grad_out.dtype not in _DTYPES:
            grad_out = grad_out.float()
        gi, gom = dcn_backward(input, offset_mask, grad_out.contiguous(), *ctx.conf)
        if input.dtype != torch.float32:
            gi = gi.to(input.dtype)
        return gi, gom, None, None, None, None, None, None


def deformable_conv(input, offset_mask, groups, kernel=3, stride=1, pad=1, dilation=1,
                    out_dtype=None):
    return DCNFunction.apply(input, offset_mask, groups, kernel, stride, pad, dilation, out_dtype)
