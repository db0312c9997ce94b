"""Pins of the fp64 oracle against facts fixed by the page and by mathematics.

Definition followed: the Sparse4D deformable_aggregation walkthrough
(mhpn.cn/news/1081857), sections 3.2 (bilinear sampling), 4.1 (gradients)
and 5.1 (sum over points, cameras, scales).  None of these tests re-types
the oracle's formula: each one checks it against an independent fact --
torch's grid_sample (the library routine the op reduces to), exact texels,
a constant map, affine maps (closed form), out-of-bounds zeros, linearity
and adjoint identities, forward probing, and finite differences.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from view_deformable_feature_amd import workloads as W

KEYS = ("feat", "spatial_shape", "scale_start_index", "loc", "weights")


def _args(inp):
    return [inp[k] for k in KEYS]


def _dyadic_loc(rng, shape, lo, hi, denom=1024):
    """Locations i/denom: binary32 and fp64 pixel coordinates then agree exactly."""
    i = rng.integers(int(np.floor(lo * denom)), int(np.ceil(hi * denom)), size=shape)
    return (i / denom).astype(np.float32)


def _small(name="small", **kw):
    base = dict(bs=2, num_cams=2, levels=((8, 12), (4, 6), (1, 3)), C=16, groups=4,
                anchors=5, pts=3, loc_lo=-0.15, loc_hi=1.15, weight_kind="uniform01",
                seed=7)
    base.update(kw)
    return W.custom(name, **base)


# --------------------------------------------------------------------------------------
# library special case: torch grid_sample(bilinear, zeros, align_corners=False), fp64
# --------------------------------------------------------------------------------------

def _grid_sample_reference(inp, requires_grad=False):
    """out[b,a,c] = sum_{p,k,s} w[b,a,p,k,s,g(c)] * grid_sample(level_ks, 2*loc-1)[c].

    Returns (out, leaves) where leaves = (feat_t, loc_t, w_t) fp64 torch tensors.
    """
    feat = torch.from_numpy(np.asarray(inp["feat"], dtype=np.float64))
    loc = torch.from_numpy(inp["loc"].astype(np.float64))
    w = torch.from_numpy(inp["weights"].astype(np.float64))
    for t in (feat, loc, w):
        t.requires_grad_(requires_grad)
    shape, start = inp["spatial_shape"], inp["scale_start_index"]
    bs, num_feat, C = feat.shape
    _, A, P, K, _ = loc.shape
    S, G = w.shape[4], w.shape[5]
    D = C // G
    out = torch.zeros(bs, A, C, dtype=torch.float64)
    for k in range(K):
        for s in range(S):
            H, Wd = int(shape[k, s, 0]), int(shape[k, s, 1])
            st = int(start[k, s])
            level = feat[:, st:st + H * Wd, :].reshape(bs, H, Wd, C).permute(0, 3, 1, 2)
            grid = (2.0 * loc[:, :, :, k, :] - 1.0).reshape(bs, A * P, 1, 2)
            smp = F.grid_sample(level, grid, mode="bilinear", padding_mode="zeros",
                                align_corners=False)             # [bs, C, A*P, 1]
            smp = smp[..., 0].permute(0, 2, 1).reshape(bs, A, P, C)
            wc = w[:, :, :, k, s, :].repeat_interleave(D, dim=-1)  # [bs, A, P, C]
            out = out + (wc * smp).sum(dim=2)
    return out, (feat, loc, w)


def _avoid_exact_minus_one(loc, shape):
    """grid_sample differs from the op only at a pixel coordinate of exactly -1 (the
    op's window is open there); nudge such dyadic locations off that line."""
    loc = loc.copy()
    K, S = shape.shape[:2]
    for k in range(K):
        for s in range(S):
            H, Wd = shape[k, s]
            for d, ext in ((0, Wd), (1, H)):
                v = loc[..., k, d]
                bad = (v.astype(np.float64) * ext - 0.5) == -1.0
                v[bad] += np.float32(1.0 / 1024)
    return loc


@pytest.mark.parametrize("seed", [0, 1])
def test_forward_matches_grid_sample(seed):
    wl = _small(seed=seed)
    inp = W.make_inputs(wl)
    rng = np.random.default_rng(seed + 50)
    inp["loc"] = _avoid_exact_minus_one(
        _dyadic_loc(rng, inp["loc"].shape, -0.15, 1.15), inp["spatial_shape"])
    ref, _ = _grid_sample_reference(inp)
    got = oracle.forward(*_args(inp))
    np.testing.assert_allclose(got, ref.numpy(), rtol=0, atol=1e-13)


def test_forward_matches_grid_sample_nuscenes_subset():
    """The nuScenes-shaped pyramid (4 scales, 6 cameras) with 12 anchors."""
    wl = W.custom("nus_sub", bs=1, num_cams=6, levels=((64, 176), (32, 88), (16, 44), (8, 22)),
                  C=16, groups=8, anchors=12, pts=13, loc_lo=-0.05, loc_hi=1.05, seed=3)
    inp = W.make_inputs(wl)
    rng = np.random.default_rng(11)
    inp["loc"] = _avoid_exact_minus_one(
        _dyadic_loc(rng, inp["loc"].shape, -0.05, 1.05), inp["spatial_shape"])
    ref, _ = _grid_sample_reference(inp)
    got = oracle.forward(*_args(inp))
    np.testing.assert_allclose(got, ref.numpy(), rtol=0, atol=1e-13)


def test_backward_matches_grid_sample_autograd():
    wl = _small(seed=4)
    inp = W.make_inputs(wl)
    rng = np.random.default_rng(99)
    inp["loc"] = _avoid_exact_minus_one(
        _dyadic_loc(rng, inp["loc"].shape, -0.15, 1.15), inp["spatial_shape"])
    out, (feat_t, loc_t, w_t) = _grid_sample_reference(inp, requires_grad=True)
    go = torch.from_numpy(inp["grad_out"].astype(np.float64))
    (out * go).sum().backward()
    gf, gl, gw = oracle.backward(*_args(inp), inp["grad_out"])
    np.testing.assert_allclose(gf, feat_t.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(gw, w_t.grad.numpy(), rtol=0, atol=1e-12)
    # torch reaches loc through grid = 2*loc - 1, which its autograd accounts for
    np.testing.assert_allclose(gl, loc_t.grad.numpy(), rtol=1e-12, atol=1e-10)


# --------------------------------------------------------------------------------------
# exact texel, constant map, affine map
# --------------------------------------------------------------------------------------

def test_exact_texel_tiny():
    """Pixel-centre locations ((j+0.5)/16, (i+0.5)/16) return feat[i, j, :] exactly."""
    wl = W.WORKLOADS["tiny"]
    inp = W.make_inputs(wl)
    H = Wd = 16
    A, P = wl.anchors, wl.pts
    rng = np.random.default_rng(5)
    ij = rng.integers(0, 16, size=(A, P, 2))
    loc = np.empty((1, A, P, 1, 2), np.float32)
    loc[0, :, :, 0, 0] = (ij[..., 1] + 0.5) / Wd
    loc[0, :, :, 0, 1] = (ij[..., 0] + 0.5) / H
    inp["loc"] = loc
    for p in range(P):
        w = np.zeros_like(inp["weights"])
        w[0, :, p] = 1.0
        inp["weights"] = w
        got = oracle.forward(*_args(inp))
        for a in range(A):
            i, j = ij[a, p]
            assert np.array_equal(got[0, a], inp["feat"][0, i * Wd + j].astype(np.float64))


def test_constant_map():
    """feat == kappa, weights summing to one per (b, a, g), all four corners inside:
    out == kappa, grad_loc == 0, grad_weights[g] == kappa * sum_{c in g} grad_out."""
    kappa = 0.8125
    wl = _small(seed=9, levels=((8, 12), (4, 6)))
    inp = W.make_inputs(wl)
    inp["feat"] = np.full_like(inp["feat"], kappa)
    w = inp["weights"].astype(np.float64)
    w /= w.sum(axis=(2, 3, 4), keepdims=True)
    inp["weights"] = w.astype(np.float32)
    wsum = inp["weights"].astype(np.float64).sum(axis=(2, 3, 4))       # [bs, A, G]
    # a location whose pixel coordinate lies in [0, H-1] x [0, W-1] at every scale:
    # inside the pixel-centre span of the coarsest level along each axis
    rng = np.random.default_rng(3)
    shape = inp["spatial_shape"]
    loc = np.empty_like(inp["loc"])
    eps = 1e-3
    for k in range(wl.num_cams):
        Hmin, Wmin = shape[k, :, 0].min(), shape[k, :, 1].min()
        loc[..., k, 0] = rng.uniform(0.5 / Wmin + eps, 1 - 0.5 / Wmin - eps, size=loc.shape[:3])
        loc[..., k, 1] = rng.uniform(0.5 / Hmin + eps, 1 - 0.5 / Hmin - eps, size=loc.shape[:3])
    inp["loc"] = loc
    out = oracle.forward(*_args(inp))
    D = wl.C // wl.groups
    np.testing.assert_allclose(out, kappa * np.repeat(wsum, D, axis=-1), rtol=0, atol=1e-14)
    _, gl, gw = oracle.backward(*_args(inp), inp["grad_out"])
    np.testing.assert_allclose(gl, 0.0, atol=1e-12)
    gsum = inp["grad_out"].astype(np.float64).reshape(wl.bs, wl.anchors, wl.groups, D).sum(-1)
    np.testing.assert_allclose(gw, np.broadcast_to(kappa * gsum[:, :, None, None, None, :], gw.shape),
                               rtol=1e-14, atol=1e-13)


def test_affine_map_closed_form():
    """Bilinear interpolation reproduces an affine map f(i, j) = al*i + be*j + ga exactly
    wherever all four corners are inside: val = al*h + be*w + ga with h = y*H - 0.5,
    w = x*W - 0.5, so d val/dx = be*W and d val/dy = al*H (location gradient scaled by
    width for x and by height for y, section 4.1).  H and W are powers of two and the
    pixel coordinates multiples of 1/64, so every input is exact in binary32."""
    H, Wd, C = 8, 16, 6
    rng = np.random.default_rng(21)
    al, be, ga = (np.round(rng.normal(size=C) * 64) / 64 for _ in range(3))
    ii, jj = np.meshgrid(np.arange(H), np.arange(Wd), indexing="ij")
    feat = (al * ii[..., None] + be * jj[..., None] + ga).reshape(1, H * Wd, C).astype(np.float32)
    A, P = 4, 5
    w_px = rng.integers(0, (Wd - 1) * 64, size=(A, P)) / 64.0   # w in [0, W-1): corners inside
    h_px = rng.integers(0, (H - 1) * 64, size=(A, P)) / 64.0
    loc = np.stack([(w_px + 0.5) / Wd, (h_px + 0.5) / H], -1)[None, :, :, None, :].astype(np.float32)
    weights = rng.random((1, A, P, 1, 1, 1), dtype=np.float32)
    shape = np.array([[[H, Wd]]], np.int32)
    start = np.zeros((1, 1), np.int32)
    out = oracle.forward(feat, shape, start, loc, weights)
    val = al * h_px[..., None] + be * w_px[..., None] + ga       # [A, P, C]
    wt = weights[0, :, :, 0, 0, 0, None].astype(np.float64)      # [A, P, 1]
    np.testing.assert_allclose(out[0], (wt * val).sum(1), rtol=1e-13, atol=1e-13)
    go = rng.standard_normal((1, A, C)).astype(np.float32)
    _, gl, gw = oracle.backward(feat, shape, start, loc, weights, go)
    top = wt * go[0, :, None, :].astype(np.float64)              # [A, P, C]
    np.testing.assert_allclose(gl[0, :, :, 0, 0], (be * Wd * top).sum(-1), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(gl[0, :, :, 0, 1], (al * H * top).sum(-1), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(gw[0, :, :, 0, 0, 0],
                               (go[0, :, None, :].astype(np.float64) * val).sum(-1),
                               rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------------------
# out of bounds
# --------------------------------------------------------------------------------------

def test_out_of_bounds_contributes_zero():
    wl = W.WORKLOADS["tiny"]
    inp = W.make_inputs(wl)
    loc = inp["loc"].copy()
    # x = -0.1 at W = 16 gives w = -2.1; y = 1.1 gives h = 17.1 >= H
    loc[0, :, 0, 0, 0] = -0.1
    loc[0, :, 1, 0, 1] = 1.1
    loc[0, :, 2, 0, 0] = -1.0 / 32     # w = -1 exactly: outside the open window
    inp["loc"] = loc
    base = oracle.forward(*_args(inp))
    gf, gl, gw = oracle.backward(*_args(inp), inp["grad_out"])
    assert np.all(gl[0, :, :3] == 0.0) and np.all(gw[0, :, :3] == 0.0)
    # changing the features or the weights of those samples changes nothing
    w2 = inp["weights"].copy()
    w2[0, :, :3] = 123.0
    alt = oracle.forward(inp["feat"], inp["spatial_shape"], inp["scale_start_index"], loc, w2)
    assert np.array_equal(base, alt)


def test_half_pixel_border_uses_one_column():
    """w in (-1, 0): only column 0 is inside, with weight lw = w + 1."""
    H, Wd, C = 4, 5, 3
    rng = np.random.default_rng(2)
    feat = rng.standard_normal((1, H * Wd, C)).astype(np.float32)
    # x = 1/64 -> w = 5/64 - 0.5 = -27/64 ; y = 3/8 -> h = 1.0 exactly
    loc = np.array([1 / 64, 3 / 8], np.float32).reshape(1, 1, 1, 1, 2)
    weights = np.ones((1, 1, 1, 1, 1, 1), np.float32)
    out = oracle.forward(feat, np.array([[[H, Wd]]], np.int32), np.zeros((1, 1), np.int32), loc, weights)
    lw = -27 / 64 + 1
    np.testing.assert_allclose(out[0, 0], lw * feat[0, 1 * Wd + 0].astype(np.float64), rtol=0, atol=1e-15)


# --------------------------------------------------------------------------------------
# linearity, homogeneity and adjoint identities
# --------------------------------------------------------------------------------------

def test_linear_in_weights_and_homogeneity():
    wl = _small(seed=12)
    inp = W.make_inputs(wl)
    rng = np.random.default_rng(1)
    w1 = inp["weights"]
    w2 = rng.standard_normal(w1.shape).astype(np.float32)
    al, be = 0.75, -1.5
    f = lambda w: oracle.forward(inp["feat"], inp["spatial_shape"], inp["scale_start_index"],
                                 inp["loc"], w)
    lhs = f((al * w1.astype(np.float64) + be * w2).astype(np.float32))
    # al*w1 + be*w2 is exact in binary32 only up to rounding: compare with tolerance
    rhs = al * f(w1) + be * f(w2)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-6, atol=1e-6)
    out = f(w1)
    gf, gl, gw = oracle.backward(*_args(inp), inp["grad_out"])
    go = inp["grad_out"].astype(np.float64)
    s_out = float((go * out).sum())
    np.testing.assert_allclose(float((gw * w1).sum()), s_out, rtol=1e-12)
    np.testing.assert_allclose(float((gf * inp["feat"]).sum()), s_out, rtol=1e-12)


def test_grad_feat_by_forward_probing():
    """out is linear in the features and channel-separable, so the forward with a
    one-hot feature row r gives d out[b,a,c] / d feat[b,r,c]; contracting with grad_out
    must give the backward's grad_feat row r (tiny workload, every row probed)."""
    wl = W.WORKLOADS["tiny"]
    inp = W.make_inputs(wl)
    gf, _, _ = oracle.backward(*_args(inp), inp["grad_out"])
    go = inp["grad_out"].astype(np.float64)
    probe = np.zeros_like(inp["feat"])
    for r in range(wl.num_feat):
        probe[:] = 0.0
        probe[0, r, :] = 1.0
        d = oracle.forward(probe, inp["spatial_shape"], inp["scale_start_index"], inp["loc"],
                           inp["weights"])
        np.testing.assert_allclose(gf[0, r], (go[0] * d[0]).sum(0), rtol=1e-13, atol=1e-14)


def test_grad_weights_by_forward_probing():
    wl = _small(seed=13)
    inp = W.make_inputs(wl)
    _, _, gw = oracle.backward(*_args(inp), inp["grad_out"])
    go = inp["grad_out"].astype(np.float64)
    P, K, S, G, C = wl.pts, wl.num_cams, wl.num_scale, wl.groups, wl.C
    D = C // G
    for p in range(P):
        for k in range(K):
            for s in range(S):
                for g in range(G):
                    w = np.zeros_like(inp["weights"])
                    w[:, :, p, k, s, g] = 1.0
                    d = oracle.forward(inp["feat"], inp["spatial_shape"],
                                       inp["scale_start_index"], inp["loc"], w)
                    expect = (go * d)[:, :, g * D:(g + 1) * D].sum(-1)
                    np.testing.assert_allclose(gw[:, :, p, k, s, g], expect, rtol=1e-13,
                                               atol=1e-14)


# --------------------------------------------------------------------------------------
# finite differences on the location
# --------------------------------------------------------------------------------------

def test_grad_loc_central_differences():
    """The interpolant is affine in x (and in y) inside a cell, so a dyadic central
    difference that crosses no grid line is exact up to fp64 rounding."""
    wl = _small(seed=17)
    inp = W.make_inputs(wl)
    rng = np.random.default_rng(8)
    denom = 1024
    inp["loc"] = _dyadic_loc(rng, inp["loc"].shape, -0.15, 1.15, denom)
    delta = 1.0 / 8192
    go = inp["grad_out"].astype(np.float64)
    _, gl, _ = oracle.backward(*_args(inp), inp["grad_out"])
    shape = inp["spatial_shape"]
    checked = 0
    for b in range(wl.bs):
        for a in range(wl.anchors):
            for p in range(wl.pts):
                for k in range(wl.num_cams):
                    for d in range(2):
                        # skip coordinates whose +-delta step meets a grid line or the
                        # window border at any scale of this camera
                        x = float(inp["loc"][b, a, p, k, d])
                        ext = shape[k, :, 0 if d == 1 else 1].astype(np.float64)
                        px = x * ext - 0.5
                        lo, hi = (x - delta) * ext - 0.5, (x + delta) * ext - 0.5
                        if np.any(np.floor(lo) != np.floor(hi)) or np.any(np.floor(px) != np.floor(lo)):
                            continue
                        lp = inp["loc"].copy()
                        lm = inp["loc"].copy()
                        lp[b, a, p, k, d] = x + delta
                        lm[b, a, p, k, d] = x - delta
                        fp = oracle.forward(inp["feat"], shape, inp["scale_start_index"], lp, inp["weights"])
                        fm = oracle.forward(inp["feat"], shape, inp["scale_start_index"], lm, inp["weights"])
                        fd = float((go[b, a] * (fp[b, a] - fm[b, a])).sum()) / (2 * delta)
                        np.testing.assert_allclose(gl[b, a, p, k, d], fd, rtol=1e-9, atol=1e-9)
                        checked += 1
    assert checked > 0.5 * gl.size


# --------------------------------------------------------------------------------------
# the sampled entry points agree with the dense ones
# --------------------------------------------------------------------------------------

def test_sampled_entry_points_match_dense():
    wl = _small(seed=23)
    inp = W.make_inputs(wl)
    out = oracle.forward(*_args(inp))
    gf, gl, gw = oracle.backward(*_args(inp), inp["grad_out"])
    ids = np.array([0, 3, wl.anchors + 1, 2 * wl.anchors - 1])
    o2 = oracle.forward(*_args(inp), anchor_ids=ids)
    assert np.array_equal(o2, out.reshape(-1, wl.C)[ids])
    gl2, gw2 = oracle.backward_anchors(*_args(inp), inp["grad_out"], ids)
    assert np.array_equal(gl2, gl.reshape(-1, *gl.shape[2:])[ids])
    assert np.array_equal(gw2, gw.reshape(-1, *gw.shape[2:])[ids])
    rows = np.array([0, 5, 17, wl.num_feat + 3, 2 * wl.num_feat - 1])
    gf2 = oracle.grad_feat_rows(*_args(inp), inp["grad_out"], rows)
    assert np.array_equal(gf2, gf.reshape(-1, wl.C)[rows])


def _torch_bf16_values(bits: np.ndarray) -> np.ndarray:
    """float32 values of bfloat16 bit patterns, widened by torch (not by this repository)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16))
    return t.view(torch.bfloat16).float().numpy()


def test_bf16_features_read_exactly():
    # bfloat16 patterns and their values (sign, 8-bit exponent biased by 127, 7-bit
    # fraction; subnormals below 2^-126)
    golden = {0x3F80: 1.0, 0xC000: -2.0, 0x7F7F: (2.0 - 2.0 ** -7) * 2.0 ** 127,
              0x0080: 2.0 ** -126, 0x0001: 2.0 ** -133, 0x3EAB: 0.333984375, 0x8000: -0.0}
    bits = np.array(list(golden), np.uint16)
    assert np.array_equal(_torch_bf16_values(bits).astype(np.float64), list(golden.values()))
    wl = W.custom("tb", bs=1, num_cams=1, levels=((16, 16),), C=32, groups=4, anchors=8,
                  pts=4, feat_dtype="bf16", loc_lo=-0.1, loc_hi=1.1, seed=31)
    inp = W.make_inputs(wl)
    as_f32 = dict(inp)
    as_f32["feat"] = _torch_bf16_values(inp["feat"])
    assert np.array_equal(oracle.forward(*_args(inp)), oracle.forward(*_args(as_f32)))
    gi = oracle.backward(*_args(inp), inp["grad_out"])
    gf = oracle.backward(*_args(as_f32), inp["grad_out"])
    for a, b in zip(gi, gf):
        assert np.array_equal(a, b)


def test_generator_bf16_rounding_matches_torch():
    """The input generator's bfloat16 rounding (used for the bf16 features) is torch's
    round-to-nearest-even, ties included: values whose low 16 bits are exactly 0x8000
    round to the even neighbour, 0x7FFF down and 0x8001 up."""
    import torch
    rng = np.random.default_rng(5)
    hi = rng.integers(0, 0x7F7F, size=4096, dtype=np.uint32)     # finite, below the top binade
    sign = rng.integers(0, 2, size=hi.size, dtype=np.uint32) << np.uint32(31)
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF], np.uint32)
    u = (sign[:, None] | (hi[:, None] << np.uint32(16)) | lows[None, :]).reshape(-1)
    x = np.concatenate([u.view(np.float32),
                        rng.standard_normal(100000).astype(np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(W.bf16_bits_from_f32(x), ref)


def test_f16_features_read_exactly():
    # IEEE binary16 patterns and their values (sign, 5-bit exponent biased by 15,
    # 10-bit fraction; subnormals below 2^-14)
    golden = {0x3C00: 1.0, 0xC000: -2.0, 0x7BFF: 65504.0, 0x0400: 2.0 ** -14,
              0x0001: 2.0 ** -24, 0x3555: 1365.0 / 4096.0, 0x8000: -0.0}
    bits = np.array(list(golden), np.uint16)
    assert np.array_equal(bits.view(np.float16).astype(np.float64), list(golden.values()))
    wl = W.custom("th", bs=1, num_cams=1, levels=((16, 16),), C=32, groups=4, anchors=8,
                  pts=4, feat_dtype="f16", loc_lo=-0.1, loc_hi=1.1, seed=32)
    inp = W.make_inputs(wl)
    assert inp["feat"].dtype == np.float16
    as_f32 = dict(inp)
    as_f32["feat"] = inp["feat"].astype(np.float32)
    assert np.array_equal(oracle.forward(*_args(inp)), oracle.forward(*_args(as_f32)))
    gf16 = oracle.backward(*_args(inp), inp["grad_out"])
    gf32 = oracle.backward(*_args(as_f32), inp["grad_out"])
    assert all(np.array_equal(a, b) for a, b in zip(gf16, gf32))
    with pytest.raises(TypeError):      # bfloat16 grad_out must arrive as its values
        oracle.backward(*_args(inp), W.bf16_bits_from_f32(inp["grad_out"]))


def test_rejects_malformed_problem():
    wl = W.WORKLOADS["tiny"]
    inp = W.make_inputs(wl)
    bad = dict(inp)
    bad["scale_start_index"] = np.array([[1]], np.int32)      # 1 + 256 > num_feat
    with pytest.raises(ValueError):
        oracle.forward(*_args(bad))


@pytest.mark.parametrize("threads", [1, 3])
def test_forward_parallel_equals_forward(threads):
    """The OpenMP forward (a timing reference only) gives the one-thread loop's
    result bit for bit: each anchor's row is formed by the same code, in the same
    order, by one thread."""
    inp = W.make_inputs(W.WORKLOADS["nuscenes_fwd"])
    args = [inp[k] for k in ("feat", "spatial_shape", "scale_start_index", "loc", "weights")]
    seq = oracle.forward(*args)
    par, used = oracle.forward_parallel(*args, threads=threads)
    assert used == threads
    assert np.array_equal(seq, par)
