"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Every workload, the full-size large ones included, is compared on every output
element; the large ones run the oracle one batch image per thread and also check
identities that hold at any size.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import (KEYS, TOL_BF16, TOL_BWD, TOL_FWD, assert_close, gpu_backward,
                         gpu_forward, say, to_device)
from view_deformable_feature_amd import workloads as W

pytestmark = pytest.mark.gpu


def _args(inp):
    return [inp[k] for k in KEYS]


# (level slices, backward form): the library's choice of both; slices forced on; the
# row-ordered backward forced; the per-anchor backward forced, with and without slices
MODES = {"auto": (None, None), "sliced": (True, None), "roworder": (None, False),
         "regather": (None, True), "regather_sliced": (True, True),
         "regather_unsliced": (False, True), "unsliced": (False, None)}


def _full_check(inp, tol_f, tol_b, label, slices=None, regather=None):
    say(f"[parity] {label}: upload")
    dev = to_device(inp)
    say(f"[parity] {label}: forward (slices={slices})")
    out = gpu_forward(dev, slices=slices).cpu().numpy()
    say(f"[parity] {label}: backward (slices={slices}, regather={regather})")
    gf, gl, gw = (t.cpu().numpy() for t in gpu_backward(dev, slices=slices, regather=regather))
    say(f"[parity] {label}: oracle")
    r_out = oracle.forward(*_args(inp))
    r_gf, r_gl, r_gw = oracle.backward(*_args(inp), inp["grad_out"])
    e = [assert_close(f"{label} out", out, r_out, tol_f),
         assert_close(f"{label} grad_feat", gf, r_gf, tol_b),
         assert_close(f"{label} grad_loc", gl, r_gl, tol_b),
         assert_close(f"{label} grad_weights", gw, r_gw, tol_b)]
    say(f"[parity] {label}: max err out {e[0]:.2e} gf {e[1]:.2e} gl {e[2]:.2e} gw {e[3]:.2e}")
    return dev, out


# ---------------------------------------------------------------------------------------
# the five workloads
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("mode", ["auto", "sliced", "roworder", "regather", "regather_sliced"])
def test_tiny_full(mode):
    inp = W.make_inputs(W.WORKLOADS["tiny"])
    _full_check(inp, TOL_FWD, TOL_BWD, "tiny", *MODES[mode])


# nuScenes-shaped workloads take level slices by default (92 MB of features, 24 levels)
@pytest.mark.parametrize("slices", [None, False], ids=["auto", "unsliced"])
def test_nuscenes_forward_full(slices):
    inp = W.make_inputs(W.WORKLOADS["nuscenes_fwd"], with_grad_out=False)
    dev = to_device(inp)
    say(f"[parity] nuscenes_fwd: forward (slices={slices})")
    out = gpu_forward(dev, slices=slices).cpu().numpy()
    ref = oracle.forward(*_args(inp))
    say(f"[parity] nuscenes_fwd max err {assert_close('nuscenes out', out, ref, TOL_FWD):.2e}")
    out2 = gpu_forward(dev, slices=slices).cpu().numpy()
    assert np.array_equal(out, out2), "forward is not deterministic"


@pytest.mark.parametrize("mode", ["auto", "regather", "regather_unsliced"])
def test_nuscenes_backward_full(mode):
    slices, regather = MODES[mode]
    inp = W.make_inputs(W.WORKLOADS["nuscenes_bwd"])
    dev = to_device(inp)
    say(f"[parity] nuscenes_bwd: backward x2 ({mode})")
    r1 = [t.cpu().numpy() for t in gpu_backward(dev, slices=slices, regather=regather)]
    r2 = [t.cpu().numpy() for t in gpu_backward(dev, slices=slices, regather=regather)]
    ref = oracle.backward(*_args(inp), inp["grad_out"])
    for run, r in (("run1", r1), ("run2", r2)):
        for name, g, rr in zip(("grad_feat", "grad_loc", "grad_weights"), r, ref):
            assert_close(f"nuscenes {run} {name}", g, rr, TOL_BWD)
    # only the atomically accumulated feature gradient may differ between runs
    assert np.array_equal(r1[1], r2[1]) and np.array_equal(r1[2], r2[2])
    say(f"[parity] nuscenes_bwd run-to-run max |d grad_feat| = "
        f"{np.abs(r1[0] - r2[0]).max():.3e}")


# The oracle of a large workload runs one batch image per thread (ctypes releases
# the GIL; each image is an independent problem with bs = 1), and is computed once per
# workload for all the backward forms compared against it.
_ORACLE_CACHE = {}


def _per_image_oracle(inp):
    from concurrent.futures import ThreadPoolExecutor
    bs = inp["feat"].shape[0]

    def image(b):
        sub = {k: inp[k][b:b + 1] for k in ("feat", "loc", "weights", "grad_out")}
        args = [sub["feat"], inp["spatial_shape"], inp["scale_start_index"], sub["loc"],
                sub["weights"]]
        return oracle.forward(*args)[0], oracle.backward(*args, sub["grad_out"])

    with ThreadPoolExecutor(max_workers=min(bs, 8)) as ex:
        res = list(ex.map(image, range(bs)))
    out = np.stack([r[0] for r in res])
    gf, gl, gw = (np.stack([r[1][i][0] for r in res]) for i in range(3))
    return out, gf, gl, gw


def _large_inputs_and_oracle(name):
    if name not in _ORACLE_CACHE:
        _ORACLE_CACHE.clear()            # one large workload held at a time
        say(f"[parity] {name}: generate")
        inp = W.make_inputs(W.WORKLOADS[name])
        say(f"[parity] {name}: oracle, one batch image per thread")
        _ORACLE_CACHE[name] = (inp, _per_image_oracle(inp))
    return _ORACLE_CACHE[name]


def _close_per_image(name, got, ref, tol):
    """assert_close one batch image at a time (bounds the temporaries)."""
    err = 0.0
    for b in range(ref.shape[0]):
        err = max(err, assert_close(f"{name} [image {b}]", got[b], ref[b], tol))
    return err


def _full_large_check(name, tol_f, tol_b, slices=None, regather=None):
    """Every element of out, grad_feat, grad_loc and grad_weights of a full-size large
    workload against the oracle; the backward runs twice and both runs must pass."""
    wl = W.WORKLOADS[name]
    inp, (r_out, r_gf, r_gl, r_gw) = _large_inputs_and_oracle(name)
    dev = to_device(inp)
    say(f"[parity] {name}: forward (slices={slices})")
    out = gpu_forward(dev, slices=slices)
    e_out = _close_per_image(f"{name} out", out.cpu().numpy(), r_out, tol_f)
    runs = []
    for run in (1, 2):
        say(f"[parity] {name}: backward run {run} (slices={slices}, regather={regather})")
        gf, gl, gw = gpu_backward(dev, slices=slices, regather=regather)
        gf_h, gl_h, gw_h = gf.cpu().numpy(), gl.cpu().numpy(), gw.cpu().numpy()
        e = (_close_per_image(f"{name} run{run} grad_feat", gf_h, r_gf, tol_b),
             _close_per_image(f"{name} run{run} grad_loc", gl_h, r_gl, tol_b),
             _close_per_image(f"{name} run{run} grad_weights", gw_h, r_gw, tol_b))
        say(f"[parity] {name} run{run}: max err out {e_out:.2e} gf {e[0]:.2e} gl {e[1]:.2e} "
            f"gw {e[2]:.2e}")
        runs.append((gf_h, gl_h, gw_h))
        del gf, gl, gw
    # only the atomically ordered feature gradient may differ between runs
    assert np.array_equal(runs[0][1], runs[1][1]) and np.array_equal(runs[0][2], runs[1][2])
    d = max(float(np.abs(runs[0][0][b] - runs[1][0][b]).max()) for b in range(wl.bs))
    say(f"[parity] {name}: run-to-run max |d grad_feat| = {d:.3e}")
    # identities at full size: <grad_out, out> = <grad_feat, feat> = <grad_weights, weights>
    go = dev["grad_out"].double()
    s_out = float((go * out.double()).sum())
    s_feat = sum(float((torch.from_numpy(runs[0][0][b]).to("cuda").double()
                        * dev["feat"][b].double()).sum()) for b in range(wl.bs))
    s_w = float((torch.from_numpy(runs[0][2]).to("cuda").double() * dev["weights"].double()).sum())
    scale = float((go.abs() * out.double().abs()).sum())
    assert abs(s_feat - s_out) <= 1e-4 * scale, (s_feat, s_out)
    assert abs(s_w - s_out) <= 1e-4 * scale, (s_w, s_out)


@pytest.mark.parametrize("mode", ["auto", "roworder", "regather_unsliced"])
def test_large_full(mode):
    _full_large_check("large", TOL_FWD, TOL_BWD, *MODES[mode])


@pytest.mark.parametrize("mode", ["auto", "roworder", "regather"])
def test_large_bf16_full(mode):
    _full_large_check("large_bf16", TOL_BF16, TOL_BF16, *MODES[mode])


# ---------------------------------------------------------------------------------------
# ragged shapes, several tiles, edge cases
# ---------------------------------------------------------------------------------------

RAGGED = [
    # (name, kwargs) -- channel counts that exercise each lane layout
    ("c96_g3", dict(bs=2, num_cams=3, levels=((13, 29), (7, 15), (3, 8)), C=96, groups=3,
                    anchors=37, pts=5, loc_lo=-0.1, loc_hi=1.1)),
    ("c48_g6", dict(bs=1, num_cams=2, levels=((11, 17), (6, 9)), C=48, groups=6, anchors=29,
                    pts=7, loc_lo=-0.2, loc_hi=1.2)),
    ("c2_g2", dict(bs=2, num_cams=1, levels=((5, 7),), C=2, groups=2, anchors=65, pts=3,
                   loc_lo=-0.2, loc_hi=1.2, weight_kind="uniform01")),
    ("c1_g1", dict(bs=1, num_cams=2, levels=((4, 6), (2, 3)), C=1, groups=1, anchors=130,
                   pts=2, loc_lo=-0.3, loc_hi=1.3)),
    ("c6_g3", dict(bs=1, num_cams=1, levels=((9, 9),), C=6, groups=3, anchors=40, pts=4,
                   loc_lo=-0.1, loc_hi=1.1)),
    ("c512_g8", dict(bs=1, num_cams=2, levels=((16, 40), (8, 20)), C=512, groups=8, anchors=21,
                     pts=6, loc_lo=-0.05, loc_hi=1.05)),
    ("c1024_g8", dict(bs=1, num_cams=1, levels=((8, 12),), C=1024, groups=8, anchors=9, pts=3,
                      loc_lo=-0.05, loc_hi=1.05)),
    ("c256_g8_many_pts", dict(bs=1, num_cams=6, levels=((12, 30), (6, 15)), C=256, groups=8,
                              anchors=5, pts=97, loc_lo=-0.05, loc_hi=1.05)),
    ("c32_g1_64_levels", dict(bs=1, num_cams=8, levels=tuple((2 + i, 3 + 2 * i) for i in range(8)),
                              C=32, groups=1, anchors=11, pts=3, loc_lo=-0.1, loc_hi=1.1)),
    ("c64_g64", dict(bs=1, num_cams=1, levels=((6, 6),), C=64, groups=64, anchors=12, pts=3,
                     loc_lo=-0.1, loc_hi=1.1)),
    ("clustered", dict(bs=2, num_cams=3, levels=((20, 50), (10, 25)), C=128, groups=4,
                       anchors=33, pts=13, loc_kind="clustered", loc_sigma=0.01)),
    # a 150x130 level (19,500 rows: counted by two row tiles) next to a 70x70 one
    # (4,900 rows: also two tiles, since tiles run) and a small one (LDS histogram)
    ("c16_g2_row_tiles", dict(bs=2, num_cams=1, levels=((150, 130), (70, 70), (9, 11)), C=16,
                              groups=2, anchors=300, pts=12, loc_lo=-0.05, loc_hi=1.05)),
    # the same with odd row counts: 19,781 rows in two tiles of 9,891 and 9,890 rows,
    # 4,899 in two of 2,450 and 2,449 (every tiled level is cut into as many tiles)
    ("c16_g2_row_tiles_odd", dict(bs=2, num_cams=1, levels=((151, 131), (71, 69), (9, 11)), C=16,
                                  groups=2, anchors=300, pts=12, loc_lo=-0.05, loc_hi=1.05)),
    # 16,800 (anchor, point) pairs per image: levels counted in LDS take 8 samples per
    # thread, 2048 per workgroup, the last chunk ragged
    ("c16_g4_count_chunks", dict(bs=2, num_cams=1, levels=((40, 90), (30, 40), (9, 11)), C=16,
                                 groups=4, anchors=2100, pts=8, loc_lo=-0.05, loc_hi=1.05)),
]


@pytest.mark.parametrize("rows_h", [1024, 1025])
def test_row_order_scan_tile_boundary(rows_h):
    """1024 x 1024 rows are 256 scan tiles, whose totals every bucket workgroup
    adds up itself; 1025 x 1024 rows are 257 tiles, added up by a separate launch.
    Row-ordered form, 1,600 samples over a million rows (most rows zeroed, the
    level counted by 64 row tiles)."""
    wl = W.custom(f"tiles_{rows_h}", bs=1, num_cams=1, levels=((rows_h, 1024),), C=4, groups=1,
                  anchors=200, pts=8, loc_lo=0.0, loc_hi=1.0, seed=90 + rows_h % 7)
    inp = W.make_inputs(wl)
    _full_check(inp, TOL_FWD, TOL_BWD, wl.name, *MODES["roworder"])


@pytest.mark.parametrize("name, kw", RAGGED, ids=[r[0] for r in RAGGED])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("mode", ["auto", "sliced", "roworder", "regather_sliced"])
def test_ragged_full(name, kw, dtype, mode):
    wl = W.custom(f"{name}_{dtype}", feat_dtype=dtype, seed=zlib.crc32(name.encode()) % 1000, **kw)
    inp = W.make_inputs(wl)
    tol_f, tol_b = (TOL_BF16, TOL_BF16) if dtype == "bf16" else (TOL_FWD, TOL_BWD)
    _full_check(inp, tol_f, tol_b, wl.name, *MODES[mode])


def test_per_camera_pyramids_and_permuted_level_order():
    """Cameras with different pyramids, levels stored scale-major in reverse order."""
    wl = W.custom("percam", bs=2, num_cams=3, levels=((9, 14), (5, 7)),
                  cam_levels=(((9, 14), (5, 7)), ((12, 10), (6, 5)), ((7, 21), (4, 11))),
                  C=64, groups=4, anchors=23, pts=6, loc_lo=-0.1, loc_hi=1.1, seed=77)
    inp = W.make_inputs(wl)
    shape, start = inp["spatial_shape"], inp["scale_start_index"]
    order = [(k, s) for s in reversed(range(wl.num_scale)) for k in reversed(range(wl.num_cams))]
    feat = inp["feat"]
    new_feat = np.empty_like(feat)
    new_start = np.zeros_like(start)
    row = 0
    for k, s in order:
        n = int(shape[k, s, 0] * shape[k, s, 1])
        new_feat[:, row:row + n] = feat[:, start[k, s]:start[k, s] + n]
        new_start[k, s] = row
        row += n
    inp2 = dict(inp, feat=new_feat, scale_start_index=new_start)
    _full_check(inp2, TOL_FWD, TOL_BWD, "permuted")


def test_golden_fixtures_on_gpu():
    from golden_fixtures import fixture_paths, load
    for path in fixture_paths():
        d, inp, exp = load(path)
        dev = to_device(inp)
        out = gpu_forward(dev).cpu().numpy()
        gf, gl, gw = (t.cpu().numpy() for t in gpu_backward(dev))
        assert_close("golden out", out, exp["out"], TOL_FWD)
        assert_close("golden grad_feat", gf, exp["grad_feat"], TOL_BWD)
        assert_close("golden grad_loc", gl, exp["grad_loc"], TOL_BWD)
        assert_close("golden grad_weights", gw, exp["grad_weights"], TOL_BWD)


def test_exact_texels_bit_exact():
    """Pixel-centre locations with one-hot weights return the stored texel exactly."""
    wl = W.WORKLOADS["tiny"]
    inp = W.make_inputs(wl)
    rng = np.random.default_rng(3)
    ij = rng.integers(0, 16, size=(wl.anchors, wl.pts, 2))
    loc = np.empty((1, wl.anchors, wl.pts, 1, 2), np.float32)
    loc[0, :, :, 0, 0] = (ij[..., 1] + 0.5) / 16
    loc[0, :, :, 0, 1] = (ij[..., 0] + 0.5) / 16
    w = np.zeros_like(inp["weights"])
    w[0, :, 1] = 1.0
    dev = to_device(dict(inp, loc=loc, weights=w))
    out = gpu_forward(dev).cpu().numpy()
    for a in range(wl.anchors):
        i, j = ij[a, 1]
        assert np.array_equal(out[0, a], inp["feat"][0, i * 16 + j])


@pytest.mark.parametrize("slices", [None, True], ids=["auto", "sliced"])
def test_no_points_and_empty_batches(slices):
    wl = W.custom("nopts", bs=2, num_cams=2, levels=((4, 5),), C=32, groups=4, anchors=3, pts=0,
                  weight_kind="uniform01")
    inp = W.make_inputs(wl)
    dev = to_device(inp)
    out = torch.full((2, 3, 32), 5.0, device="cuda")
    import view_deformable_feature_amd as vdf
    vdf.da_forward(dev["feat"], dev["spatial_shape"], dev["scale_start_index"], dev["loc"],
                   dev["weights"], out=out, slices=slices)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out) == 0
    gf = torch.full(tuple(dev["feat"].shape), 7.0, device="cuda")
    gf, gl, gw = vdf.da_backward(dev["feat"], dev["spatial_shape"], dev["scale_start_index"],
                                 dev["loc"], dev["weights"], dev["grad_out"], grad_feat=gf,
                                 slices=slices)
    torch.cuda.synchronize()
    assert torch.count_nonzero(gf) == 0 and gl.numel() == 0 and gw.numel() == 0
    for kw in (dict(anchors=0, pts=4), dict(bs=0, anchors=3, pts=4)):
        wl = W.custom("empty", num_cams=2, levels=((4, 5),), C=32, groups=4,
                      **dict(dict(bs=1), **kw))
        inp = W.make_inputs(wl)
        dev = to_device(inp)
        out = gpu_forward(dev, slices=slices)
        gf, gl, gw = gpu_backward(dev, slices=slices)
        assert out.numel() == 0 and gl.numel() == 0 and gw.numel() == 0
        assert torch.count_nonzero(gf) == 0


@pytest.mark.parametrize("mode", ["auto", "sliced", "roworder", "regather"])
def test_nan_and_far_locations_contribute_nothing(mode):
    wl = W.custom("nanloc", bs=1, num_cams=2, levels=((8, 8), (4, 4)), C=32, groups=2,
                  anchors=10, pts=4, loc_lo=-0.1, loc_hi=1.1, seed=5)
    inp = W.make_inputs(wl)
    loc = inp["loc"].copy()
    loc[0, :, 0, :, 0] = np.nan
    loc[0, :, 1, :, 1] = np.inf
    loc[0, :, 2, :, :] = -3e38
    inp["loc"] = loc
    _full_check(inp, TOL_FWD, TOL_BWD, "nanloc", *MODES[mode])


def test_max_extent_levels():
    """Levels at DA_MAX_EXTENT along one axis."""
    wl = W.custom("maxext", bs=1, num_cams=1, levels=((32768, 1),), C=8, groups=2,
                  anchors=40, pts=8, loc_lo=-0.05, loc_hi=1.05, seed=9,
                  cam_levels=None)
    inp = W.make_inputs(wl)
    _full_check(inp, TOL_FWD, TOL_BWD, "maxext_h")
    wl = W.custom("maxext_w", bs=1, num_cams=1, levels=((1, 32768),), C=8, groups=2,
                  anchors=40, pts=8, loc_lo=-0.05, loc_hi=1.05, seed=10)
    _full_check(W.make_inputs(wl), TOL_FWD, TOL_BWD, "maxext_w")


@pytest.mark.parametrize("mode", ["auto", "sliced", "roworder", "regather"])
def test_accumulate_adds_into_existing_gradient(mode):
    slices, regather = MODES[mode]
    inp = W.make_inputs(W.custom("acc", bs=1, num_cams=2, levels=((10, 12), (5, 6)), C=64,
                                 groups=4, anchors=17, pts=5, loc_lo=-0.1, loc_hi=1.1, seed=12))
    dev = to_device(inp)
    base = torch.randn(tuple(dev["feat"].shape), device="cuda", generator=None)
    gf0, gl0, gw0 = gpu_backward(dev, slices=slices, regather=regather)
    gf1, gl1, gw1 = gpu_backward(dev, accumulate_into=base.clone(), slices=slices,
                                 regather=regather)
    assert_close("accumulate", gf1.cpu().numpy(), (base + gf0).cpu().numpy(), 1e-6)
    assert torch.equal(gl0, gl1) and torch.equal(gw0, gw1)


def test_autograd_function_and_side_stream():
    import view_deformable_feature_amd as vdf
    inp = W.make_inputs(W.custom("ag", bs=2, num_cams=2, levels=((9, 11), (5, 6)), C=64,
                                 groups=8, anchors=14, pts=4, loc_lo=-0.1, loc_hi=1.1, seed=21))
    dev = to_device(inp)
    feat = dev["feat"].clone().requires_grad_(True)
    loc = dev["loc"].clone().requires_grad_(True)
    w = dev["weights"].clone().requires_grad_(True)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out = vdf.DeformableAggregationFunction.apply(feat, inp["spatial_shape"],
                                                      torch.from_numpy(inp["scale_start_index"]),
                                                      loc, w)
        out.backward(dev["grad_out"])
    torch.cuda.synchronize()
    r_out = oracle.forward(*_args(inp))
    r_gf, r_gl, r_gw = oracle.backward(*_args(inp), inp["grad_out"])
    assert_close("autograd out", out.detach().cpu().numpy(), r_out, TOL_FWD)
    assert_close("autograd grad_feat", feat.grad.cpu().numpy(), r_gf, TOL_BWD)
    assert_close("autograd grad_loc", loc.grad.cpu().numpy(), r_gl, TOL_BWD)
    assert_close("autograd grad_weights", w.grad.cpu().numpy(), r_gw, TOL_BWD)


def test_errors_surface_as_exceptions():
    import view_deformable_feature_amd as vdf
    from view_deformable_feature_amd._lib import DAError
    inp = W.make_inputs(W.WORKLOADS["tiny"])
    dev = to_device(inp)
    bad_start = np.array([[5]], np.int32)
    with pytest.raises(DAError, match="inside num_feat"):
        vdf.da_forward(dev["feat"], dev["spatial_shape"], bad_start, dev["loc"], dev["weights"])


# ---------------------------------------------------------------------------------------
# the scatter form and workspace handling
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny", "nuscenes_bwd"])
def test_backward_atomic_form(name):
    inp = W.make_inputs(W.WORKLOADS[name])
    dev = to_device(inp)
    say(f"[parity] {name}: da_backward_atomic")
    gf, gl, gw = (t.cpu().numpy() for t in gpu_backward(dev, atomic=True))
    r_gf, r_gl, r_gw = oracle.backward(*_args(inp), inp["grad_out"])
    assert_close(f"{name} atomic grad_feat", gf, r_gf, TOL_BWD)
    assert_close(f"{name} atomic grad_loc", gl, r_gl, TOL_BWD)
    assert_close(f"{name} atomic grad_weights", gw, r_gw, TOL_BWD)


def test_backward_atomic_form_ragged_bf16():
    wl = W.custom("atomic_ragged", bs=2, num_cams=3, levels=((13, 29), (7, 15)), C=96, groups=3,
                  anchors=19, pts=5, feat_dtype="bf16", loc_lo=-0.1, loc_hi=1.1, seed=41)
    inp = W.make_inputs(wl)
    dev = to_device(inp)
    gf, gl, gw = (t.cpu().numpy() for t in gpu_backward(dev, atomic=True))
    r_gf, r_gl, r_gw = oracle.backward(*_args(inp), inp["grad_out"])
    assert_close("atomic bf16 grad_feat", gf, r_gf, TOL_BF16)
    assert_close("atomic bf16 grad_loc", gl, r_gl, TOL_BF16)
    assert_close("atomic bf16 grad_weights", gw, r_gw, TOL_BF16)


@pytest.mark.parametrize("mode", ["auto", "sliced", "roworder", "regather"])
def test_workspace_reused_across_calls(mode):
    """One caller-owned workspace serves two calls in a row, the second smaller; its
    stale contents from the first call must not leak into the second.  Same for the
    forward's workspace."""
    import view_deformable_feature_amd as vdf
    slices, regather = MODES[mode]
    big = W.make_inputs(W.custom("ws_big", bs=2, num_cams=2, levels=((20, 30), (10, 15)), C=64,
                                 groups=4, anchors=40, pts=7, loc_lo=-0.1, loc_hi=1.1, seed=51))
    small = W.make_inputs(W.custom("ws_small", bs=1, num_cams=2, levels=((6, 9), (3, 5)), C=64,
                                   groups=4, anchors=9, pts=3, loc_lo=-0.1, loc_hi=1.1, seed=52))
    dev_b, dev_s = to_device(big), to_device(small)
    n = vdf.workspace_size(dev_b["feat"], dev_b["spatial_shape"], dev_b["loc"], dev_b["weights"],
                           regather=regather)
    ws = torch.full((n,), 0xAB, dtype=torch.uint8, device="cuda")
    nf = vdf.forward_workspace_size(dev_b["feat"], dev_b["spatial_shape"], dev_b["loc"],
                                    dev_b["weights"], slices=slices)
    fws = torch.full((max(nf, 1),), 0xAB, dtype=torch.uint8, device="cuda")
    for inp, dev in ((big, dev_b), (small, dev_s), (big, dev_b)):
        out = gpu_forward(dev, slices=slices, workspace=fws).cpu().numpy()
        assert_close("ws out", out, oracle.forward(*_args(inp)), TOL_FWD)
        gf, gl, gw = (t.cpu().numpy() for t in gpu_backward(dev, workspace=ws, slices=slices,
                                                             regather=regather))
        r_gf, r_gl, r_gw = oracle.backward(*_args(inp), inp["grad_out"])
        assert_close("ws grad_feat", gf, r_gf, TOL_BWD)
        assert_close("ws grad_loc", gl, r_gl, TOL_BWD)
        assert_close("ws grad_weights", gw, r_gw, TOL_BWD)


@pytest.mark.parametrize("mode", ["auto", "sliced", "roworder", "regather"])
def test_hot_rows_span_many_chunks(mode):
    """A 2x3 level hit by 4000 samples: each of its rows collects thousands of
    feature-gradient terms, far more than one wave's chunk of the row-sorted list,
    next to a large level with a few terms per row."""
    wl = W.custom("hot_rows", bs=2, num_cams=2, levels=((2, 3), (40, 60)), C=64, groups=4,
                  anchors=250, pts=8, loc_lo=0.0, loc_hi=1.0, seed=61)
    inp = W.make_inputs(wl)
    _full_check(inp, TOL_FWD, TOL_BWD, "hot_rows", *MODES[mode])


# ---------------------------------------------------------------------------------------
# deterministic backward
# ---------------------------------------------------------------------------------------

DET_CASES = [
    ("nuscenes_bwd", None),
    ("hot_rows", dict(bs=2, num_cams=2, levels=((2, 3), (40, 60)), C=64, groups=4, anchors=250,
                      pts=8, loc_lo=0.0, loc_hi=1.0, seed=61)),
    ("c96_g3_bf16", dict(bs=2, num_cams=3, levels=((13, 29), (7, 15), (3, 8)), C=96, groups=3,
                         anchors=37, pts=5, loc_lo=-0.1, loc_hi=1.1, feat_dtype="bf16", seed=7)),
    # 256 scan tiles: the bucket kernel adds up the tile totals and reduces the bounds
    ("tiles_256", dict(bs=1, num_cams=1, levels=((1024, 1024),), C=4, groups=1, anchors=200,
                       pts=8, loc_lo=0.0, loc_hi=1.0, seed=63)),
    # levels counted by row tiles (two per tiled level, ragged) beside an LDS-counted one
    ("row_tiles", dict(bs=2, num_cams=1, levels=((151, 131), (71, 69), (9, 11)), C=16, groups=2,
                       anchors=300, pts=12, loc_lo=-0.05, loc_hi=1.05, seed=62)),
]


@pytest.mark.parametrize("name, kw", DET_CASES, ids=[c[0] for c in DET_CASES])
def test_deterministic_backward_is_bit_identical(name, kw):
    """grad_feat is the same bit for bit across runs, backward forms and level slices
    (64-bit fixed-point row sums), and within the tolerance of the oracle."""
    wl = W.WORKLOADS[name] if kw is None else W.custom(name, **kw)
    inp = W.make_inputs(wl)
    dev = to_device(inp)
    say(f"[det] {name}")
    runs = []
    for slices, regather in ((None, None), (None, None), (None, True), (True, True), (False, False),
                             (True, False)):
        gf, gl, gw = gpu_backward(dev, slices=slices, regather=regather, deterministic=True)
        runs.append((gf.cpu().numpy(), gl.cpu().numpy(), gw.cpu().numpy()))
    for r in runs[1:]:
        assert np.array_equal(r[0], runs[0][0]), "deterministic grad_feat differs"
    ref = oracle.backward(*_args(inp), inp["grad_out"])
    tol = TOL_BF16 if wl.feat_dtype == "bf16" else TOL_BWD
    for gname, g, rr in zip(("grad_feat", "grad_loc", "grad_weights"), runs[0], ref):
        assert_close(f"det {name} {gname}", g, rr, tol)


def test_deterministic_accumulate():
    inp = W.make_inputs(W.custom("detacc", bs=1, num_cams=2, levels=((3, 4), (20, 30)), C=64,
                                 groups=4, anchors=120, pts=6, loc_lo=0.0, loc_hi=1.0, seed=71))
    dev = to_device(inp)
    base = torch.randn(tuple(dev["feat"].shape), device="cuda")
    gf0, _, _ = gpu_backward(dev, deterministic=True)
    outs = [gpu_backward(dev, accumulate_into=base.clone(), deterministic=True, regather=rg)[0]
            for rg in (None, True)]
    assert torch.equal(outs[0], outs[1])
    assert_close("det accumulate", outs[0].cpu().numpy(), (base + gf0).cpu().numpy(), 1e-6)


# ---------------------------------------------------------------------------------------
# grad_feat only 4-byte aligned: the gather falls back to one channel per lane
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("variant", ["backward", "accumulate", "deterministic"])
@pytest.mark.parametrize("mode", ["auto", "regather"])
def test_grad_feat_misaligned_by_one_float(variant, mode):
    """grad_feat at a 4-byte but not 16-byte aligned address (a view one float into a
    buffer), C = 256 and G = 8: every channel of every row must still be written."""
    import view_deformable_feature_amd as vdf
    slices, regather = MODES[mode]
    wl = W.custom("gf_misaligned", bs=2, num_cams=2, levels=((12, 20), (6, 10)), C=256,
                  groups=8, anchors=30, pts=5, loc_lo=-0.1, loc_hi=1.1, seed=83)
    inp = W.make_inputs(wl)
    dev = to_device(inp)
    shape = tuple(dev["feat"].shape)
    n = int(np.prod(shape))
    buf = torch.full((n + 1,), float("nan"), device="cuda")
    gf = buf[1:].view(shape)
    assert gf.data_ptr() % 16 == 4
    base = torch.randn(shape, device="cuda")
    args = (dev["feat"], dev["spatial_shape"], dev["scale_start_index"], dev["loc"],
            dev["weights"], dev["grad_out"])
    det = variant == "deterministic"
    if variant == "accumulate":
        gf.copy_(base)
        vdf.da_backward_accumulate(*args, gf, slices=slices, regather=regather)
    else:
        vdf.da_backward(*args, grad_feat=gf, slices=slices, regather=regather, deterministic=det)
    torch.cuda.synchronize()
    r_gf, _, _ = oracle.backward(*_args(inp), inp["grad_out"])
    got = gf.cpu().numpy()
    if variant == "accumulate":
        got = got - base.cpu().numpy()
    assert_close(f"misaligned grad_feat ({variant}, {mode})", got, r_gf,
                 TOL_BWD if variant != "accumulate" else 2 * TOL_BWD)
    assert torch.isnan(buf[:1]).all(), "the float before grad_feat was overwritten"
