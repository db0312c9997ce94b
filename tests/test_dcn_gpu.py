"""GPU parity of the deformable convolution (include/dcn.h) against the fp64
oracle (oracle/dcn_oracle.c): every output element on small and ragged shapes,
the full 56x56x128 batch-64 shape of the DCNv4 notes, 16-bit inputs and outputs,
and the edge cases of the definition (positions outside the image, NaN offsets,
an empty batch, a 1x1 kernel).

Tolerances, per element |gpu - ref| <= tol * (1 + |ref|): forward 1e-4, backward
1e-3 (binary32 arithmetic; 16-bit inputs convert exactly, so the same bounds); an
out stored in 16 bits adds half an ulp (2^-8 bfloat16, 2^-11 binary16).
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import TOL_BWD, TOL_FWD, TOL_OUT_BF16, TOL_OUT_F16, assert_close, say
from view_deformable_feature_amd import workloads as W

pytestmark = pytest.mark.gpu

CASES = {
    "tiny": dict(N=1, H=7, W=9, C=16, groups=2),
    "s2": dict(N=2, H=9, W=8, C=12, groups=3, stride=(2, 2)),
    "k35_dil": dict(N=1, H=9, W=11, C=24, groups=2, kernel=(3, 5), stride=(1, 2), pad=(1, 2),
                    dilation=(2, 1)),
    "k1": dict(N=2, H=6, W=5, C=8, groups=1, kernel=(1, 1), pad=(0, 0)),
    "c6_g6": dict(N=1, H=10, W=7, C=6, groups=6),                  # one channel per group
    "c40_g5": dict(N=2, H=8, W=8, C=40, groups=5),                 # D = 8
    "c96_g3": dict(N=1, H=12, W=13, C=96, groups=3),               # D = 32, G * Lg = 24 lanes
    "c256_g2": dict(N=1, H=6, W=7, C=256, groups=2),               # D = 128: 32 lanes per group
    "c512_g16": dict(N=1, H=5, W=6, C=512, groups=16),             # two groups per lane
    "far": dict(N=1, H=8, W=8, C=16, groups=4, offset_sigma=6.0),  # many positions outside
    "d3_pad3": dict(N=1, H=11, W=10, C=32, groups=4, pad=(3, 3), dilation=(3, 3)),
    # several tiles with ragged right and bottom edges, at stride 2
    "tiles_s2": dict(N=2, H=37, W=45, C=64, groups=4, stride=(2, 2)),
    # a 5x5 kernel with dilation 2 (the generic tap loop) across several tiles
    "k5_d2": dict(N=1, H=29, W=35, C=32, groups=2, kernel=(5, 5), pad=(4, 4), dilation=(2, 2)),
    # offsets of sigma 15 px: most corners leave the image or go to the far list
    "far_all": dict(N=1, H=40, W=40, C=16, groups=2, offset_sigma=15.0),
    # 32 channels per group (the fixed tile shape): 12 taps (three groups of four
    # taps per shared record pass), 25 taps (more than the shared form takes: the
    # general tap loop at the fixed shape), and stride 2 across several tiles
    "k34_d32": dict(N=1, H=19, W=23, C=64, groups=2, kernel=(3, 4), pad=(1, 2), seed=3100),
    "k55_d32": dict(N=1, H=17, W=21, C=32, groups=1, kernel=(5, 5), pad=(2, 2), seed=3101),
    "s2_d32": dict(N=2, H=20, W=34, C=128, groups=4, stride=(2, 2), seed=3102),
    # fewer taps than the lanes of a group (one and three: lanes without a tap)
    "k1_d32": dict(N=1, H=13, W=30, C=64, groups=2, kernel=(1, 1), pad=(0, 0), seed=3103),
    "k13_d32": dict(N=1, H=11, W=21, C=32, groups=1, kernel=(1, 3), pad=(0, 1), seed=3104),
}
_SEEDED = [n for n in sorted(CASES) if "seed" not in CASES[n]]


def _wl(name, **over):
    kw = dict(CASES[name])
    if "seed" not in kw:
        kw["seed"] = 3000 + _SEEDED.index(name)
    kw.update(over)
    return W.dcn_custom(name, **kw)


def _dev(inp):
    x = inp["input"]
    if x.dtype == np.uint16:
        xt = torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    else:
        xt = torch.from_numpy(x).cuda()
    return xt, torch.from_numpy(inp["offset_mask"]).cuda()


def _conf(wl):
    return dict(groups=wl.groups, kernel=wl.kernel, stride=wl.stride, pad=wl.pad,
                dilation=wl.dilation)


def _check(wl, out_dtype=None, go_dtype=torch.float32):
    import view_deformable_feature_amd as vdf
    inp = W.make_dcn_inputs(wl)
    x, om = _dev(inp)
    say(f"[dcn] {wl.name} {wl.dtype} out={out_dtype} go={go_dtype}")
    out = vdf.dcn_forward(x, om, **_conf(wl), out_dtype=out_dtype)
    go_t = torch.from_numpy(inp["grad_out"]).cuda().to(go_dtype)
    gi, gom = vdf.dcn_backward(x, om, go_t, **_conf(wl))
    torch.cuda.synchronize()
    ref = oracle.dcn_forward(inp["input"], inp["offset_mask"], **_conf(wl))
    tol = {None: TOL_FWD, torch.float32: TOL_FWD, torch.bfloat16: TOL_OUT_BF16,
           torch.float16: TOL_OUT_F16}[out_dtype]
    e0 = assert_close(f"{wl.name} out", out.float().cpu().numpy(), ref, tol)
    r_gi, r_gom = oracle.dcn_backward(inp["input"], inp["offset_mask"],
                                      go_t.float().cpu().numpy(), **_conf(wl))
    e1 = assert_close(f"{wl.name} grad_input", gi.cpu().numpy(), r_gi, TOL_BWD)
    e2 = assert_close(f"{wl.name} grad_offset_mask", gom.cpu().numpy(), r_gom, TOL_BWD)
    say(f"[dcn] {wl.name}: max err out {e0:.2e} gi {e1:.2e} gom {e2:.2e}")
    return x, om, out, gi, gom


@pytest.mark.parametrize("name", sorted(CASES))
def test_dcn_full(name):
    _check(_wl(name))


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("name", ["tiny", "c96_g3", "c512_g16", "k35_dil", "k34_d32"])
def test_dcn_16bit_input(name, dtype):
    _check(_wl(name, dtype=dtype))


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
def test_dcn_16bit_out_and_grad_out(out_dtype):
    wl = _wl("c40_g5")
    x, om, out16, _, _ = _check(wl, out_dtype=out_dtype, go_dtype=out_dtype)
    import view_deformable_feature_amd as vdf
    out32 = vdf.dcn_forward(x, om, **_conf(wl))
    torch.cuda.synchronize()
    assert torch.equal(out16, out32.to(out_dtype)), "16-bit out is not RNE(binary32 out)"


def test_dcn_forward_deterministic_and_offset_grads_repeatable():
    import view_deformable_feature_amd as vdf
    wl = _wl("c96_g3")
    inp = W.make_dcn_inputs(wl)
    x, om = _dev(inp)
    go = torch.from_numpy(inp["grad_out"]).cuda()
    o1 = vdf.dcn_forward(x, om, **_conf(wl))
    o2 = vdf.dcn_forward(x, om, **_conf(wl))
    g1 = vdf.dcn_backward(x, om, go, **_conf(wl))
    g2 = vdf.dcn_backward(x, om, go, **_conf(wl))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.equal(g1[1], g2[1])


def test_dcn_nan_and_far_offsets():
    import view_deformable_feature_amd as vdf
    wl = _wl("tiny")
    inp = W.make_dcn_inputs(wl)
    om = inp["offset_mask"].copy()
    K = wl.K
    hits = [(0, 1, 2, 1, 0, np.nan), (0, 3, 3, 0, 1, 1e6), (0, 6, 8, 1, 8, -1e30),
            (0, 0, 0, 0, 4, 0.999)]          # the last one stays inside
    for n, h, w, g, t, v in hits:
        om[n, h, w, g, 2 * t] = v
    inp2 = dict(inp, offset_mask=om)
    x, omt = _dev(inp2)
    out = vdf.dcn_forward(x, omt, **_conf(wl))
    go = torch.from_numpy(inp["grad_out"]).cuda()
    gi, gom = vdf.dcn_backward(x, omt, go, **_conf(wl))
    torch.cuda.synchronize()
    assert_close("nan out", out.cpu().numpy(), oracle.dcn_forward(inp["input"], om, **_conf(wl)),
                 TOL_FWD)
    r_gi, r_gom = oracle.dcn_backward(inp["input"], om, inp["grad_out"], **_conf(wl))
    assert_close("nan grad_input", gi.cpu().numpy(), r_gi, TOL_BWD)
    assert_close("nan grad_om", gom.cpu().numpy(), r_gom, TOL_BWD)
    for n, h, w, g, t, v in hits[:3]:
        assert float(gom[n, h, w, g, 2 * K + t]) == 0.0


def test_dcn_empty_batch():
    import view_deformable_feature_amd as vdf
    x = torch.zeros((0, 5, 5, 8), device="cuda")
    om = torch.zeros((0, 5, 5, 2, 27), device="cuda")
    out = vdf.dcn_forward(x, om, 2)
    gi, gom = vdf.dcn_backward(x, om, torch.zeros((0, 5, 5, 8), device="cuda"), 2)
    torch.cuda.synchronize()
    assert out.shape == (0, 5, 5, 8) and gi.shape == x.shape and gom.shape == om.shape


def test_dcn_56_full_size():
    """The DCNv4 notes' kernel ablation shape: 56x56x128, batch 64, 4 groups."""
    _check(W.DCN_WORKLOADS["dcn_56"])


def test_dcn_autograd():
    import view_deformable_feature_amd as vdf
    wl = _wl("c40_g5", dtype="f16")
    inp = W.make_dcn_inputs(wl)
    x, om = _dev(inp)
    x = x.clone().requires_grad_(True)
    om = om.clone().requires_grad_(True)
    out = vdf.deformable_conv(x, om, **_conf(wl), out_dtype=torch.bfloat16)
    g = torch.from_numpy(inp["grad_out"]).cuda()
    (out.float() * g).sum().backward()
    torch.cuda.synchronize()
    assert out.dtype == torch.bfloat16 and x.grad.dtype == torch.float16
    gi, gom = vdf.dcn_backward(x.detach(), om.detach(), g.to(torch.bfloat16), **_conf(wl))
    torch.cuda.synchronize()
    assert torch.equal(om.grad, gom)
    assert_close("autograd grad_input", x.grad.float().cpu().numpy(),
                 gi.to(torch.float16).float().cpu().numpy(), 1e-3)


@pytest.mark.parametrize("name", ["dcn_28", "dcn_14", "dcn_56_f16"])
def test_dcn_other_page_shapes_full_size(name):
    """The DCNv4 notes' other input sizes (28x28x256, 14x14x512) and the 56x56x128
    shape with binary16 input, every element against the oracle."""
    _check(W.DCN_WORKLOADS[name])


def test_dcn_grad_input_repeatable_without_far_corners():
    """Tile sums are 64-bit fixed point: with every offset inside the ring margin
    (no far corner), grad_input is the same bit for bit run after run."""
    import view_deformable_feature_amd as vdf
    wl = _wl("c96_g3", offset_sigma=0.5)
    inp = W.make_dcn_inputs(wl)
    om = inp["offset_mask"].copy()
    K = wl.K
    om[..., :2 * K] = np.clip(om[..., :2 * K], -3.5, 3.5)
    x, omt = _dev(dict(inp, offset_mask=om))
    go = torch.from_numpy(inp["grad_out"]).cuda()
    runs = [vdf.dcn_backward(x, omt, go, **_conf(wl))[0].cpu() for _ in range(3)]
    torch.cuda.synchronize()
    assert all(torch.equal(runs[0], r) for r in runs[1:])
    r_gi, _ = oracle.dcn_backward(inp["input"], om, inp["grad_out"], **_conf(wl))
    assert_close("repeatable grad_input", runs[0].numpy(), r_gi, TOL_BWD)


@pytest.mark.parametrize("C, G", [(64, 2), (64, 4)], ids=["d32_fixed_tiles", "d16_general"])
def test_dcn_offsets_at_the_ring_margin(C, G):
    """Offsets at and around the 4-pixel ring margin of the tile backward (and whole
    pixels, where a corner falls exactly on a tile edge): a sample with
    |offset| <= 4 reaches every tile that owns one of its corners through that
    tile's ring, a larger one lists its far corners.  Every element against the
    oracle, across ragged 8 x 16 tiles."""
    import view_deformable_feature_amd as vdf
    wl = W.dcn_custom("margin", N=1, H=24, W=40, C=C, groups=G, seed=3200)
    inp = W.make_dcn_inputs(wl)
    om = inp["offset_mask"].copy()
    K = wl.K
    vals = np.array([-5.0, -4.5, -4.0001, -4.0, -3.9999, -1.0, -0.5, 0.0, 0.5, 1.0,
                     3.9999, 4.0, 4.0001, 4.5, 5.0], dtype=np.float32)
    rng = np.random.default_rng(3201)
    om[..., :2 * K] = rng.choice(vals, size=om[..., :2 * K].shape)
    x, omt = _dev(dict(inp, offset_mask=om))
    go = torch.from_numpy(inp["grad_out"]).cuda()
    out = vdf.dcn_forward(x, omt, **_conf(wl))
    gi, gom = vdf.dcn_backward(x, omt, go, **_conf(wl))
    torch.cuda.synchronize()
    ref = oracle.dcn_forward(inp["input"], om, **_conf(wl))
    r_gi, r_gom = oracle.dcn_backward(inp["input"], om, inp["grad_out"], **_conf(wl))
    assert_close("margin out", out.cpu().numpy(), ref, TOL_FWD)
    assert_close("margin grad_input", gi.cpu().numpy(), r_gi, TOL_BWD)
    assert_close("margin grad_offset_mask", gom.cpu().numpy(), r_gom, TOL_BWD)


def test_dcn_unaligned_views():
    """input, offset_mask and grad_out as views one element into larger buffers: one
    channel per lane vector, the bound kernel's element-wise scans and element-wise
    grad_out loads, each against the oracle."""
    import view_deformable_feature_amd as vdf
    wl = _wl("c40_g5")
    inp = W.make_dcn_inputs(wl)
    x, om = _dev(inp)
    go = torch.from_numpy(inp["grad_out"]).cuda()

    def shifted(t):
        buf = torch.zeros(t.numel() + 1, device="cuda", dtype=t.dtype)
        v = buf[1:].view(t.shape)
        v.copy_(t)
        return v

    xv, omv, gov = shifted(x), shifted(om), shifted(go)
    assert xv.data_ptr() % 16 and omv.data_ptr() % 16 and gov.data_ptr() % 16
    say("[dcn] unaligned views c40_g5")
    out = vdf.dcn_forward(xv, omv, **_conf(wl))
    gi, gom = vdf.dcn_backward(xv, omv, gov, **_conf(wl))
    torch.cuda.synchronize()
    assert_close("unaligned out", out.cpu().numpy(),
                 oracle.dcn_forward(inp["input"], inp["offset_mask"], **_conf(wl)), TOL_FWD)
    r_gi, r_gom = oracle.dcn_backward(inp["input"], inp["offset_mask"], inp["grad_out"],
                                      **_conf(wl))
    assert_close("unaligned grad_input", gi.cpu().numpy(), r_gi, TOL_BWD)
    assert_close("unaligned grad_om", gom.cpu().numpy(), r_gom, TOL_BWD)


def test_dcn_hand_worked_golden():
    """The hand-worked problem of tests/golden/hand_dcn_1x2_taps_two_groups.json
    through the HIP path, against its printed values."""
    import json
    import os
    import view_deformable_feature_amd as vdf
    path = os.path.join(os.path.dirname(__file__), "golden", "hand_dcn_1x2_taps_two_groups.json")
    with open(path) as f:
        g = json.load(f)
    conf = dict(groups=g["groups"], kernel=tuple(g["kernel"]), stride=tuple(g["stride"]),
                pad=tuple(g["pad"]), dilation=tuple(g["dilation"]))
    x = torch.tensor(g["input"], dtype=torch.float32, device="cuda")
    om = torch.tensor(g["offset_mask"], dtype=torch.float32, device="cuda")
    go = torch.tensor(g["grad_out"], dtype=torch.float32, device="cuda")
    say("[dcn] hand-worked golden")
    out = vdf.dcn_forward(x, om, **conf)
    gi, gom = vdf.dcn_backward(x, om, go, **conf)
    torch.cuda.synchronize()
    assert_close("golden out", out.cpu().numpy(), np.array(g["expect_out"]), TOL_FWD)
    assert_close("golden grad_input", gi.cpu().numpy(), np.array(g["expect_grad_input"]), TOL_BWD)
    assert_close("golden grad_om", gom.cpu().numpy(), np.array(g["expect_grad_offset_mask"]),
                 TOL_BWD)
