"""A whole step (da_forward then da_backward; dcn_forward then dcn_backward)
captured in a HIP graph and replayed: every replay must reproduce the eager
call.

The library launches kernels only (no allocation, memset or synchronisation),
so one captured step can be replayed; each replay here follows eager work on
the same buffers (they are overwritten with NaN first) and a synchronisation.
Outputs whose arithmetic order is fixed (out, grad_loc, grad_weights, and
grad_feat of the deterministic form) must match the eager call bit for bit;
grad_feat of the default form sums long rows with atomics, so it is compared
within the backward tolerance.
"""
import numpy as np
import pytest
import torch

import view_deformable_feature_amd as vdf
from view_deformable_feature_amd import workloads as W
from gpu_helpers import TOL_BWD, assert_close, say, to_device

pytestmark = pytest.mark.gpu

RAGGED = dict(bs=2, num_cams=3, levels=((13, 29), (7, 15), (3, 8)), C=96, groups=3, anchors=37,
              pts=5, loc_lo=-0.1, loc_hi=1.1, seed=91)

# (name, custom shape or None, deterministic, backward form: None = library's choice,
#  True = per-anchor)
CASES = [
    ("nuscenes_bwd", None, False, None),
    ("nuscenes_bwd", None, True, None),
    ("ragged_c96_g3", RAGGED, False, None),
    ("ragged_c96_g3_per_anchor", RAGGED, False, True),
]


@pytest.mark.parametrize("name, kw, det, regather", CASES,
                         ids=[f"{c[0]}{'_det' if c[2] else ''}" for c in CASES])
def test_graph_replays_match_eager(name, kw, det, regather):
    wl = W.WORKLOADS[name] if kw is None else W.custom(name, **kw)
    inp = W.make_inputs(wl)
    dev = to_device(inp)
    feat, loc, w, go = dev["feat"], dev["loc"], dev["weights"], dev["grad_out"]
    shape, start = dev["spatial_shape"], dev["scale_start_index"]
    out = torch.empty((wl.bs, wl.anchors, wl.C), device="cuda", dtype=torch.float32)
    gf = torch.empty(tuple(feat.shape), device="cuda", dtype=torch.float32)
    gl = torch.empty(tuple(loc.shape), device="cuda", dtype=torch.float32)
    gw = torch.empty(tuple(w.shape), device="cuda", dtype=torch.float32)
    fws_n = vdf.forward_workspace_size(feat, shape, loc, w)
    fws = torch.empty(fws_n, device="cuda", dtype=torch.uint8) if fws_n else None
    bws = torch.empty(vdf.workspace_size(feat, shape, loc, w, regather=regather,
                                         deterministic=det), device="cuda", dtype=torch.uint8)

    def step():
        vdf.da_forward(feat, shape, start, loc, w, out=out, workspace=fws)
        vdf.da_backward(feat, shape, start, loc, w, go, grad_feat=gf, grad_loc=gl,
                        grad_weights=gw, workspace=bws, regather=regather, deterministic=det)

    say(f"[graph] {name} det={det} regather={regather}: eager")
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (out, gf, gl, gw)]

    # warm up on a side stream, then capture one step
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for r in range(4):
        for t in (out, gf, gl, gw):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        say(f"[graph] {name}: replay {r}")
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref[0]), f"replay {r}: out differs from the eager call"
        assert torch.equal(gl, ref[2]), f"replay {r}: grad_loc differs from the eager call"
        assert torch.equal(gw, ref[3]), f"replay {r}: grad_weights differs from the eager call"
        if det:
            assert torch.equal(gf, ref[1]), f"replay {r}: grad_feat differs from the eager call"
        else:
            assert_close(f"graph replay {r} grad_feat", gf.cpu().numpy(),
                         ref[1].cpu().numpy().astype(np.float64), TOL_BWD)
    del graph


# deformable convolution: forward then backward, captured and replayed the same way;
# out and grad_offset_mask have a fixed arithmetic order, grad_input adds its far
# corners with atomics and is compared within the backward tolerance
DCN_CASES = [
    ("dcn_56", None),
    ("tiles_s2", dict(N=2, H=37, W=45, C=64, groups=4, stride=(2, 2), seed=3101)),
]


@pytest.mark.parametrize("name, kw", DCN_CASES, ids=[c[0] for c in DCN_CASES])
def test_dcn_graph_replays_match_eager(name, kw):
    wl = W.DCN_WORKLOADS[name] if kw is None else W.dcn_custom(name, **kw)
    inp = W.make_dcn_inputs(wl)
    x = torch.from_numpy(inp["input"]).cuda()
    om = torch.from_numpy(inp["offset_mask"]).cuda()
    go = torch.from_numpy(inp["grad_out"]).cuda()
    conf = dict(groups=wl.groups, kernel=wl.kernel, stride=wl.stride, pad=wl.pad,
                dilation=wl.dilation)
    out = torch.empty(tuple(go.shape), device="cuda", dtype=torch.float32)
    gi = torch.empty(tuple(x.shape), device="cuda", dtype=torch.float32)
    gom = torch.empty_like(om)
    nws = vdf.dcn_workspace_size(x, **conf)
    ws = torch.empty(nws, device="cuda", dtype=torch.uint8) if nws else None

    def step():
        vdf.dcn_forward(x, om, **conf, out=out)
        vdf.dcn_backward(x, om, go, **conf, grad_input=gi, grad_offset_mask=gom, workspace=ws)

    say(f"[graph] {name}: eager")
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (out, gi, gom)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for r in range(4):
        for t in (out, gi, gom):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        say(f"[graph] {name}: replay {r}")
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref[0]), f"replay {r}: out differs from the eager call"
        assert torch.equal(gom, ref[2]), f"replay {r}: grad_offset_mask differs from the eager call"
        assert_close(f"graph replay {r} grad_input", gi.cpu().numpy(),
                     ref[1].cpu().numpy().astype(np.float64), TOL_BWD)
    del graph


def test_device_level_tables_are_copied_once_and_capture_cleanly():
    """Level tables held as device tensors (as a model keeps them) are copied to the
    host on first use only: the same unchanged tensor is served from the binding's
    cache (no blocking copy, so the call can be captured), an in-place update through
    torch is seen, and the results equal those of host tables bit for bit."""
    from view_deformable_feature_amd.api import _host_i32
    wl = W.custom("devtables", **RAGGED)
    inp = W.make_inputs(wl)
    dev = to_device(inp)
    feat, loc, w, go = dev["feat"], dev["loc"], dev["weights"], dev["grad_out"]
    d_shape = torch.from_numpy(inp["spatial_shape"]).cuda()
    d_start = torch.from_numpy(inp["scale_start_index"]).cuda()
    first = _host_i32(d_start)
    assert _host_i32(d_start) is first and np.array_equal(first, inp["scale_start_index"])
    bumped = d_start.clone()
    bumped.add_(0)                                     # same values, new version
    assert np.array_equal(_host_i32(bumped), first)
    d_start.add_(1)
    assert np.array_equal(_host_i32(d_start), inp["scale_start_index"] + 1)
    d_start.sub_(1)

    ref_out = vdf.da_forward(feat, inp["spatial_shape"], inp["scale_start_index"], loc, w)
    ref_gf, ref_gl, ref_gw = vdf.da_backward(feat, inp["spatial_shape"], inp["scale_start_index"],
                                             loc, w, go)
    out = torch.empty_like(ref_out)
    gf, gl, gw = torch.empty_like(ref_gf), torch.empty_like(ref_gl), torch.empty_like(ref_gw)
    fws_n = vdf.forward_workspace_size(feat, inp["spatial_shape"], loc, w)
    fws = torch.empty(fws_n, device="cuda", dtype=torch.uint8) if fws_n else None
    bws = torch.empty(vdf.workspace_size(feat, inp["spatial_shape"], loc, w, deterministic=True),
                      device="cuda", dtype=torch.uint8)

    def step():
        vdf.da_forward(feat, d_shape, d_start, loc, w, out=out, workspace=fws)
        vdf.da_backward(feat, d_shape, d_start, loc, w, go, grad_feat=gf, grad_loc=gl,
                        grad_weights=gw, workspace=bws, deterministic=True)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                         # warms the table cache
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):                      # a blocking copy here would raise
        step()
    for _ in range(2):
        out.fill_(float("nan"))
        gf.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out)
        assert torch.equal(gl, ref_gl) and torch.equal(gw, ref_gw)
        assert_close("device tables grad_feat", gf.cpu().numpy(), ref_gf.cpu().numpy(), TOL_BWD)
    del graph
