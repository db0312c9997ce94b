"""Pins of the deformable-convolution oracle (oracle/dcn_oracle.c) against what
the DCNv4 notes and the mathematics fix, using independent library routines:

* zero offsets: the operator is a depthwise convolution whose 3x3 (or kh x kw)
  kernel holds the modulation scalars -- torch's conv2d with groups = C, with
  stride, padding and dilation;
* fractional offsets: each (group, tap) term is bilinear sampling -- torch's
  grid_sample (align_corners=True maps pixel indices exactly, zero padding);
* gradients: torch autograd through that grid_sample formulation, fp64;
* identities of a bilinear form: <grad_out, out> = <grad_mask, mask> =
  <grad_input, input>;
* out-of-image and NaN positions contribute nothing; 16-bit inputs are read as
  their exact values.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from view_deformable_feature_amd import workloads as W

CFGS = [
    # N, H, W, C, G, kernel, stride, pad, dilation
    (2, 7, 9, 12, 3, (3, 3), (1, 1), (1, 1), (1, 1)),
    (1, 8, 6, 8, 8, (3, 3), (2, 2), (1, 1), (1, 1)),
    (1, 9, 11, 6, 2, (3, 5), (1, 2), (1, 2), (2, 1)),
    (2, 5, 5, 4, 1, (1, 1), (1, 1), (0, 0), (1, 1)),
    (1, 6, 7, 10, 5, (2, 3), (1, 1), (0, 1), (1, 1)),
    (1, 10, 12, 6, 3, (3, 3), (1, 1), (2, 2), (2, 3)),
]
IDS = [f"N{c[0]}_{c[1]}x{c[2]}_C{c[3]}_G{c[4]}_k{c[5][0]}{c[5][1]}_s{c[6][0]}{c[6][1]}"
       f"_p{c[7][0]}{c[7][1]}_d{c[8][0]}{c[8][1]}" for c in CFGS]


def _out_hw(H, W, k, s, p, d):
    return ((H + 2 * p[0] - d[0] * (k[0] - 1) - 1) // s[0] + 1,
            (W + 2 * p[1] - d[1] * (k[1] - 1) - 1) // s[1] + 1)


def _draw(cfg, seed, sigma=0.7, zero_offsets=False):
    N, H, W_, C, G, k, s, p, d = cfg
    rng = np.random.default_rng(seed)
    ho, wo = _out_hw(H, W_, k, s, p, d)
    K = k[0] * k[1]
    x = rng.standard_normal((N, H, W_, C)).astype(np.float32)
    om = np.empty((N, ho, wo, G, 3 * K), np.float32)
    om[..., :2 * K] = 0.0 if zero_offsets else rng.normal(0, sigma, (N, ho, wo, G, 2 * K))
    om[..., 2 * K:] = rng.uniform(-1, 1, (N, ho, wo, G, K))
    go = rng.standard_normal((N, ho, wo, C)).astype(np.float32)
    return x, om, go


def _call(fn, cfg, *a):
    N, H, W_, C, G, k, s, p, d = cfg
    return fn(*a, groups=G, kernel=k, stride=s, pad=p, dilation=d)


@pytest.mark.parametrize("cfg", CFGS, ids=IDS)
def test_zero_offsets_is_depthwise_conv(cfg):
    N, H, W_, C, G, k, s, p, d = cfg
    K, D = k[0] * k[1], C // G
    x, om, _ = _draw(cfg, 1, zero_offsets=True)
    m = np.random.default_rng(2).uniform(-1, 1, (G, K)).astype(np.float32)
    om[..., 2 * K:] = m                              # the same scalars at every pixel
    out = _call(oracle.dcn_forward, cfg, x, om)
    weight = torch.from_numpy(np.repeat(m, D, axis=0).reshape(C, 1, k[0], k[1])).double()
    ref = F.conv2d(torch.from_numpy(x).double().permute(0, 3, 1, 2), weight, stride=s,
                   padding=p, dilation=d, groups=C).permute(0, 2, 3, 1).numpy()
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def _torch_dcn(x, om, cfg, grad=False):
    """The operator as a sum of grid_sample terms, fp64 (positions rounded to
    binary32 like the definition, offsets still differentiable)."""
    N, H, W_, C, G, k, s, p, d = cfg
    K, D = k[0] * k[1], C // G
    ho, wo = om.shape[1:3]
    xt = torch.from_numpy(x).double().requires_grad_(grad)
    omt = torch.from_numpy(om).double().requires_grad_(grad)
    gy, gx = torch.meshgrid(torch.arange(ho) * s[0] - p[0], torch.arange(wo) * s[1] - p[1],
                            indexing="ij")
    out = torch.zeros((N, C, ho, wo), dtype=torch.float64)
    for g in range(G):
        xg = xt[..., g * D:(g + 1) * D].permute(0, 3, 1, 2)
        for t in range(K):
            i, j = divmod(t, k[1])
            dx, dy = omt[:, :, :, g, 2 * t], omt[:, :, :, g, 2 * t + 1]
            bx = (gx + j * d[1]).double()
            by = (gy + i * d[0]).double()
            # binary32 position, gradient 1 in the offset
            px32 = (bx.float() + dx.detach().float()).double()
            py32 = (by.float() + dy.detach().float()).double()
            px = px32 + (dx - dx.detach())
            py = py32 + (dy - dy.detach())
            grid = torch.stack([2 * px / (W_ - 1) - 1, 2 * py / (H - 1) - 1], dim=-1)
            v = F.grid_sample(xg, grid, mode="bilinear", padding_mode="zeros",
                              align_corners=True)
            out[:, g * D:(g + 1) * D] += omt[:, :, :, g, 2 * K + t][:, None] * v
    return xt, omt, out.permute(0, 2, 3, 1)


@pytest.mark.parametrize("cfg", CFGS[:3] + CFGS[4:], ids=IDS[:3] + IDS[4:])
def test_fractional_offsets_match_grid_sample(cfg):
    x, om, _ = _draw(cfg, 3)
    out = _call(oracle.dcn_forward, cfg, x, om)
    _, _, ref = _torch_dcn(x, om, cfg)
    np.testing.assert_allclose(out, ref.detach().numpy(), rtol=0, atol=1e-11)


@pytest.mark.parametrize("cfg", CFGS[:3] + CFGS[4:], ids=IDS[:3] + IDS[4:])
def test_backward_matches_autograd(cfg):
    x, om, go = _draw(cfg, 4)
    gi, gom = _call(oracle.dcn_backward, cfg, x, om, go)
    xt, omt, ref = _torch_dcn(x, om, cfg, grad=True)
    (ref * torch.from_numpy(go).double()).sum().backward()
    np.testing.assert_allclose(gi, xt.grad.numpy(), rtol=0, atol=1e-10)
    np.testing.assert_allclose(gom, omt.grad.numpy(), rtol=0, atol=1e-10)


def test_bilinear_identities():
    cfg = CFGS[0]
    x, om, go = _draw(cfg, 5)
    K = 9
    out = _call(oracle.dcn_forward, cfg, x, om)
    gi, gom = _call(oracle.dcn_backward, cfg, x, om, go)
    s_out = float((go.astype(np.float64) * out).sum())
    s_m = float((gom[..., 2 * K:] * om[..., 2 * K:].astype(np.float64)).sum())
    s_in = float((gi * x.astype(np.float64)).sum())
    assert abs(s_out - s_m) <= 1e-9 * (1 + abs(s_out))
    assert abs(s_out - s_in) <= 1e-9 * (1 + abs(s_out))
    # doubling every scalar doubles out
    om2 = om.copy()
    om2[..., 2 * K:] *= 2
    np.testing.assert_allclose(_call(oracle.dcn_forward, cfg, x, om2), 2 * out, rtol=0, atol=1e-12)


def test_far_and_nan_positions_contribute_nothing():
    cfg = CFGS[0]
    x, om, go = _draw(cfg, 6)
    K = 9
    bad = om.copy()
    bad[0, 1, 2, 1, 0] = 1e4           # tap 0 of group 1: far right
    bad[0, 3, 3, 0, 3] = -50.0         # tap 1 of group 0: far up
    bad[1, 2, 4, 2, 4] = np.nan        # tap 2 of group 2: NaN dx
    ref_om = om.copy()
    for (n, h, w, g, t) in ((0, 1, 2, 1, 0), (0, 3, 3, 0, 1), (1, 2, 4, 2, 2)):
        ref_om[n, h, w, g, 2 * K + t] = 0.0          # the same as a zero scalar
    out = _call(oracle.dcn_forward, cfg, x, bad)
    np.testing.assert_array_equal(out, _call(oracle.dcn_forward, cfg, x, ref_om))
    gi, gom = _call(oracle.dcn_backward, cfg, x, bad, go)
    gi2, _ = _call(oracle.dcn_backward, cfg, x, ref_om, go)
    np.testing.assert_array_equal(gi, gi2)
    for (n, h, w, g, t) in ((0, 1, 2, 1, 0), (0, 3, 3, 0, 1), (1, 2, 4, 2, 2)):
        assert gom[n, h, w, g, 2 * t] == 0 and gom[n, h, w, g, 2 * t + 1] == 0
        assert gom[n, h, w, g, 2 * K + t] == 0


def test_exact_pixel_hits_and_single_corner_border():
    # a 2x2 image, one channel: integer positions read pixels exactly; a position
    # half a pixel above the image reads half of the top row
    x = np.array([[[[1.0], [2.0]], [[3.0], [4.0]]]], np.float32)
    cfg = (1, 2, 2, 1, 1, (1, 1), (1, 1), (0, 0), (1, 1))
    om = np.zeros((1, 2, 2, 1, 3), np.float32)
    om[..., 2] = 1.0
    np.testing.assert_array_equal(_call(oracle.dcn_forward, cfg, x, om)[0, ..., 0], [[1, 2], [3, 4]])
    om[0, 0, 0, 0, :2] = (0.5, -0.5)    # position (y, x) = (-0.5, 0.5)
    got = _call(oracle.dcn_forward, cfg, x, om)[0, 0, 0, 0]
    assert got == pytest.approx(0.5 * (0.5 * 1.0 + 0.5 * 2.0), abs=1e-15)


def test_16bit_inputs_read_exactly():
    wl = W.dcn_custom("dcn16", N=1, H=6, W=7, C=8, groups=2, dtype="f16", seed=7)
    inp = W.make_dcn_inputs(wl)
    a = oracle.dcn_forward(inp["input"], inp["offset_mask"], 2)
    b = oracle.dcn_forward(inp["input"].astype(np.float32), inp["offset_mask"], 2)
    np.testing.assert_array_equal(a, b)
    bits = W.bf16_bits_from_f32(inp["input"].astype(np.float32))
    c = oracle.dcn_forward(bits, inp["offset_mask"], 2)
    d = oracle.dcn_forward(W.bf16_bits_to_f32(bits), inp["offset_mask"], 2)
    np.testing.assert_array_equal(c, d)


def test_rejects_malformed():
    x = np.zeros((1, 4, 4, 6), np.float32)
    with pytest.raises(ValueError):
        oracle.dcn_forward(x, np.zeros((1, 4, 4, 4, 27), np.float32), 4)   # 6 % 4 != 0
    with pytest.raises(ValueError):
        oracle.dcn_forward(x, np.zeros((1, 4, 4, 2, 26), np.float32), 2)   # bad last dim
    with pytest.raises(ValueError):
        oracle.dcn_out_size(2, 2, kernel=5, pad=0)


def _golden_dcn():
    import json
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "hand_dcn_1x2_taps_two_groups.json")
    with open(path) as f:
        g = json.load(f)
    conf = dict(groups=g["groups"], kernel=tuple(g["kernel"]), stride=tuple(g["stride"]),
                pad=tuple(g["pad"]), dilation=tuple(g["dilation"]))
    arr = {k: np.array(g[k], dtype=np.float32) for k in ("input", "offset_mask", "grad_out")}
    return g, conf, arr


def test_hand_worked_golden():
    """tests/golden/hand_dcn_1x2_taps_two_groups.json: a 1x2-tap, stride-2, two-group
    problem worked by hand (affine and bilinear channels, a position in (-1, 0) with
    one corner in the image, a position past the right border); every value is exact
    in binary64."""
    g, conf, a = _golden_dcn()
    out = oracle.dcn_forward(a["input"], a["offset_mask"], **conf)
    gi, gom = oracle.dcn_backward(a["input"], a["offset_mask"], a["grad_out"], **conf)
    assert np.array_equal(out, np.array(g["expect_out"]))
    assert np.array_equal(gi, np.array(g["expect_grad_input"]))
    assert np.array_equal(gom, np.array(g["expect_grad_offset_mask"]))
