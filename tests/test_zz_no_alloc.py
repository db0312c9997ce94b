"""da_backward_noalloc (the backward whose workspace is the library's static scratch
array) against da_backward with a caller workspace, through the C ABI.

Two calls in a row share the array, the second on a smaller problem, so stale
contents of the first must not leak into the second; then the deterministic form.
grad_loc and grad_weights (and grad_feat of the deterministic form) are
deterministic sums and must match bit for bit; the default grad_feat is summed in
an order that depends on atomics and must match within the backward tolerance.
"""
import ctypes

import numpy as np
import pytest
import torch

from gpu_helpers import TOL_BWD, assert_close, say, to_device
from view_deformable_feature_amd import _lib, workloads as W
from view_deformable_feature_amd.api import problem_of

pytestmark = pytest.mark.gpu


def _noalloc(dev, deterministic=False):
    """Call da_backward_noalloc directly; outputs start as NaN so that every element
    must be written."""
    lib = _lib.load()
    feat, loc, w, go = dev["feat"], dev["loc"], dev["weights"], dev["grad_out"]
    shape = np.ascontiguousarray(dev["spatial_shape"], np.int32)
    start = np.ascontiguousarray(dev["scale_start_index"], np.int32)
    prob = problem_of(feat, shape, loc, w, deterministic=deterministic)
    gf = torch.full(tuple(feat.shape), float("nan"), device="cuda")
    gl = torch.full(tuple(loc.shape), float("nan"), device="cuda")
    gw = torch.full(tuple(w.shape), float("nan"), device="cuda")
    i32p = ctypes.POINTER(ctypes.c_int32)
    vp = ctypes.c_void_p
    st = lib.da_backward_noalloc(ctypes.byref(prob), vp(feat.data_ptr()),
                                 shape.ctypes.data_as(i32p), start.ctypes.data_as(i32p),
                                 vp(loc.data_ptr()), vp(w.data_ptr()), vp(go.data_ptr()),
                                 vp(gf.data_ptr()), vp(gl.data_ptr()), vp(gw.data_ptr()),
                                 vp(torch.cuda.current_stream().cuda_stream))
    _lib.check(st, "da_backward_noalloc")
    torch.cuda.synchronize()
    return gf, gl, gw


def _reference(dev, deterministic=False):
    import view_deformable_feature_amd as vdf
    r = vdf.da_backward(dev["feat"], dev["spatial_shape"], dev["scale_start_index"], dev["loc"],
                        dev["weights"], dev["grad_out"], deterministic=deterministic)
    torch.cuda.synchronize()
    return r


def _compare(label, got, ref, deterministic):
    gf, gl, gw = (t.cpu().numpy() for t in got)
    rf, rl, rw = (t.cpu().numpy() for t in ref)
    assert np.array_equal(gl, rl), f"{label}: grad_loc differs"
    assert np.array_equal(gw, rw), f"{label}: grad_weights differs"
    if deterministic:
        assert np.array_equal(gf, rf), f"{label}: deterministic grad_feat differs"
    else:
        err = assert_close(f"{label} grad_feat", gf, rf, TOL_BWD)
        say(f"[noalloc] {label}: max |d grad_feat| vs da_backward {err:.2e}")


def test_noalloc_matches_da_backward_on_two_calls_in_a_row():
    big = W.make_inputs(W.WORKLOADS["nuscenes_bwd"])
    small = W.make_inputs(W.custom("noalloc_small", bs=2, num_cams=3, levels=((13, 29), (7, 15)),
                                   C=96, groups=3, anchors=37, pts=5, loc_lo=-0.1, loc_hi=1.1,
                                   seed=91))
    for label, inp in (("nuscenes_bwd", big), ("small after large", small)):
        dev = to_device(inp)
        say(f"[noalloc] {label}")
        _compare(label, _noalloc(dev), _reference(dev), False)
    for label, inp in (("nuscenes_bwd deterministic", big),
                       ("small deterministic after large", small)):
        dev = to_device(inp)
        say(f"[noalloc] {label}")
        _compare(label, _noalloc(dev, True), _reference(dev, True), True)


def test_noalloc_refuses_a_problem_beyond_its_scratch():
    """The 4-image 160x400 workload needs more than the array: DA_ERR_UNSUPPORTED, with
    the outputs untouched."""
    wl = W.WORKLOADS["large"]
    lib = _lib.load()
    feat = torch.zeros((wl.bs, wl.num_feat, wl.C), device="cuda")
    loc = torch.zeros((wl.bs, wl.anchors, wl.pts, wl.num_cams, 2), device="cuda")
    w = torch.zeros((wl.bs, wl.anchors, wl.pts, wl.num_cams, len(wl.levels), wl.groups),
                    device="cuda")
    go = torch.zeros((wl.bs, wl.anchors, wl.C), device="cuda")
    gl = torch.full(tuple(loc.shape), 3.0, device="cuda")
    shape, start = W.level_table(wl)
    prob = problem_of(feat, shape, loc, w)
    i32p = ctypes.POINTER(ctypes.c_int32)
    vp = ctypes.c_void_p
    st = lib.da_backward_noalloc(ctypes.byref(prob), vp(feat.data_ptr()),
                                 shape.ctypes.data_as(i32p), start.ctypes.data_as(i32p),
                                 vp(loc.data_ptr()), vp(w.data_ptr()), vp(go.data_ptr()),
                                 vp(feat.data_ptr()), vp(gl.data_ptr()), vp(w.data_ptr()),
                                 vp(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert st == _lib.DA_ERR_UNSUPPORTED
    assert torch.all(gl == 3.0)
