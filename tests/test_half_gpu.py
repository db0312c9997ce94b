"""GPU parity of the 16-bit paths: binary16 features, out written in bfloat16 /
binary16, and a 16-bit grad_out in every backward form.

Binary16 features convert to binary32 exactly, so the oracle takes the same
values and the binary32 tolerances hold.  A 16-bit out is the binary32 out
rounded once to nearest even: checked bit for bit against torch's CPU conversion
of the binary32 out of the same launch configuration, and against the oracle within
the forward bound plus that rounding.  A 16-bit grad_out converts exactly, so
the backward must equal the one given those values in binary32.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import (KEYS, TOL_BF16, TOL_BWD, TOL_FWD, TOL_OUT_BF16, TOL_OUT_F16,
                         assert_close, gpu_backward, gpu_forward, say, to_device)
from view_deformable_feature_amd import workloads as W

pytestmark = pytest.mark.gpu

MODES = {"auto": (None, None), "sliced": (True, None), "roworder": (None, False),
         "regather": (None, True), "regather_sliced": (True, True)}

F16_CASES = {
    "tiny_f16": dict(bs=1, num_cams=1, levels=((16, 16),), C=32, groups=1, anchors=8, pts=4,
                     loc_lo=-0.1, loc_hi=1.1, weight_kind="uniform01", feat_dtype="f16",
                     seed=81),
    "ragged_c96_g3_f16": dict(bs=2, num_cams=3, levels=((13, 29), (7, 15), (3, 8)), C=96,
                              groups=3, anchors=37, pts=5, loc_lo=-0.1, loc_hi=1.1,
                              feat_dtype="f16", seed=82),
    "c64_g4_f16": dict(bs=2, num_cams=2, levels=((20, 30), (10, 15)), C=64, groups=4,
                       anchors=120, pts=6, loc_lo=0.0, loc_hi=1.0, feat_dtype="f16", seed=83),
}


def _args(inp):
    return [inp[k] for k in KEYS]


def _wl(name):
    return W.WORKLOADS[name] if name in W.WORKLOADS else W.custom(name, **F16_CASES[name])


def _round_out(out_f32: np.ndarray, dtype: torch.dtype) -> np.ndarray:
    """torch's CPU conversion of binary32 values to dtype (round to nearest, ties to
    even), as float64 -- a rounding implemented independently of this repository."""
    return torch.from_numpy(out_f32).to(dtype).to(torch.float64).numpy()


def _half(x: np.ndarray, dtype: torch.dtype):
    """(device tensor of x rounded to dtype, the rounded values as float32)."""
    t = torch.from_numpy(x).cuda().to(dtype)
    return t, t.float().cpu().numpy()


@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("case", list(F16_CASES))
def test_f16_features_full(case, mode):
    slices, regather = MODES[mode]
    inp = W.make_inputs(_wl(case))
    assert inp["feat"].dtype == np.float16
    dev = to_device(inp)
    assert dev["feat"].dtype == torch.float16
    say(f"[f16] {case} {mode}")
    out = gpu_forward(dev, slices=slices).cpu().numpy()
    gf, gl, gw = (t.cpu().numpy() for t in gpu_backward(dev, slices=slices, regather=regather))
    r_out = oracle.forward(*_args(inp))
    r_gf, r_gl, r_gw = oracle.backward(*_args(inp), inp["grad_out"])
    assert_close(f"{case} out", out, r_out, TOL_FWD)
    assert_close(f"{case} grad_feat", gf, r_gf, TOL_BWD)
    assert_close(f"{case} grad_loc", gl, r_gl, TOL_BWD)
    assert_close(f"{case} grad_weights", gw, r_gw, TOL_BWD)


@pytest.mark.parametrize("mode", ["auto", "regather"])
def test_nuscenes_f16_full(mode):
    slices, regather = MODES[mode]
    inp = W.make_inputs(W.WORKLOADS["nuscenes_f16"])
    dev = to_device(inp)
    say(f"[f16] nuscenes_f16 {mode}")
    out = gpu_forward(dev, slices=slices).cpu().numpy()
    gf, gl, gw = (t.cpu().numpy() for t in gpu_backward(dev, slices=slices, regather=regather))
    assert_close("nuscenes_f16 out", out, oracle.forward(*_args(inp)), TOL_FWD)
    ref = oracle.backward(*_args(inp), inp["grad_out"])
    for name, g, r in zip(("grad_feat", "grad_loc", "grad_weights"), (gf, gl, gw), ref):
        assert_close(f"nuscenes_f16 {name}", g, r, TOL_BWD)


OUT_CASES = [("nuscenes_fwd", True), ("nuscenes_fwd", False), ("tiny_f16", None),
             ("ragged_c96_g3_f16", None), ("ragged_c96_g3_bf16", None)]


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
@pytest.mark.parametrize("case, slices", OUT_CASES,
                         ids=[f"{c}-{'auto' if s is None else ('sliced' if s else 'unsliced')}"
                              for c, s in OUT_CASES])
def test_out_rounded_once(case, slices, out_dtype):
    if case == "ragged_c96_g3_bf16":
        wl = W.custom(case, **dict(F16_CASES["ragged_c96_g3_f16"], feat_dtype="bf16"))
    else:
        wl = _wl(case)
    inp = W.make_inputs(wl, with_grad_out=False)
    dev = to_device(inp)
    say(f"[out] {case} slices={slices} {out_dtype}")
    out32 = gpu_forward(dev, slices=slices).cpu().numpy()
    outh = gpu_forward(dev, slices=slices, out_dtype=out_dtype)
    assert outh.dtype == out_dtype
    got = outh.float().cpu().numpy().astype(np.float64)
    # the binary32 sums, rounded once to nearest even
    assert np.array_equal(got, _round_out(out32, out_dtype)), "16-bit out is not RNE(binary32 out)"
    tol = TOL_OUT_BF16 if out_dtype == torch.bfloat16 else TOL_OUT_F16
    if wl.feat_dtype == "bf16":
        tol += TOL_BF16
    assert_close(f"{case} out {out_dtype}", got, oracle.forward(*_args(inp)), tol)
    # a preallocated 16-bit out is written in place
    dst = torch.full_like(outh, float("nan"))
    import view_deformable_feature_amd as vdf
    vdf.da_forward(dev["feat"], dev["spatial_shape"], dev["scale_start_index"], dev["loc"],
                   dev["weights"], out=dst, slices=slices)
    torch.cuda.synchronize()
    assert torch.equal(dst, outh)


GO_MODES = ["auto", "regather", "sliced", "atomic", "deterministic"]


@pytest.mark.parametrize("go_dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
@pytest.mark.parametrize("mode", GO_MODES)
@pytest.mark.parametrize("case", ["c64_g4_f16", "nuscenes_bwd"])
def test_half_grad_out_backward(case, mode, go_dtype):
    wl = _wl(case)
    inp = W.make_inputs(wl)
    dev = to_device(inp)
    go_h, go_vals = _half(inp["grad_out"], go_dtype)
    kw = dict(slices=True if mode == "sliced" else None,
              regather=True if mode == "regather" else None,
              atomic=mode == "atomic", deterministic=mode == "deterministic")
    say(f"[grad_out] {case} {mode} {go_dtype}")
    dev32 = dict(dev, grad_out=torch.from_numpy(go_vals).cuda())
    r32 = [t.cpu().numpy() for t in gpu_backward(dev32, **kw)]
    rh = [t.cpu().numpy() for t in gpu_backward(dict(dev, grad_out=go_h), **kw)]
    # the conversion is exact: the same gradients as with binary32 grad_out
    assert np.array_equal(rh[1], r32[1]) and np.array_equal(rh[2], r32[2])
    if mode == "deterministic":
        assert np.array_equal(rh[0], r32[0])
    ref = oracle.backward(*_args(inp), go_vals)
    for name, g, r in zip(("grad_feat", "grad_loc", "grad_weights"), rh, ref):
        assert_close(f"{case} {mode} {name}", g, r, TOL_BWD)


def test_autograd_with_16bit_out():
    import view_deformable_feature_amd as vdf
    inp = W.make_inputs(W.custom("autograd16", **F16_CASES["c64_g4_f16"]))
    dev = to_device(inp)
    feat = dev["feat"].clone().requires_grad_(True)
    loc = dev["loc"].clone().requires_grad_(True)
    w = dev["weights"].clone().requires_grad_(True)
    out = vdf.deformable_aggregation(feat, dev["spatial_shape"], dev["scale_start_index"], loc, w,
                                     out_dtype=torch.bfloat16)
    assert out.dtype == torch.bfloat16
    g = torch.from_numpy(inp["grad_out"]).cuda()
    (out.float() * g).sum().backward()
    torch.cuda.synchronize()
    assert feat.grad.dtype == torch.float16
    gf, gl, gw = vdf.da_backward(dev["feat"], dev["spatial_shape"], dev["scale_start_index"],
                                 dev["loc"], dev["weights"], g.to(torch.bfloat16))
    torch.cuda.synchronize()
    assert torch.equal(loc.grad, gl) and torch.equal(w.grad, gw)
    assert_close("autograd grad_feat", feat.grad.float().cpu().numpy(),
                 gf.to(torch.float16).float().cpu().numpy(), 1e-3)
