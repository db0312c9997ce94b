"""GPU parity of level packing (section 6 of the Sparse4D walkthrough,
feature_maps_format) through the C ABI: bit-exact against the oracle's
numpy definition, in both directions, on ragged shapes and the nuScenes
pyramid; and gradients through packing feeding the aggregation."""
import zlib

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import KEYS, TOL_BWD, TOL_FWD, assert_close, say
from view_deformable_feature_amd import workloads as W

pytestmark = pytest.mark.gpu

CASES = [
    # (name, B, N, C, [(H, W) per scale])
    ("tiny", 1, 1, 4, [(2, 3)]),
    ("ragged_c", 2, 3, 70, [(13, 29), (7, 15), (3, 8)]),
    ("c1", 1, 2, 1, [(5, 7), (1, 1)]),
    ("c300", 1, 2, 300, [(9, 11), (5, 6)]),
    ("many_scales", 1, 8, 32, [(2 + i, 3 + 2 * i) for i in range(8)]),
    ("wide", 2, 1, 64, [(1, 1000), (1000, 1)]),
    ("nuscenes", 1, 6, 256, [(64, 176), (32, 88), (16, 44), (8, 22)]),
]


def _maps_np(name, B, N, C, hw, dtype):
    rng = np.random.default_rng(zlib.crc32(name.encode()) % 1000)
    if dtype == "f32":
        return [rng.standard_normal((B, N, C, h, w)).astype(np.float32) for h, w in hw]
    if dtype == "f16":
        return [rng.standard_normal((B, N, C, h, w)).astype(np.float16) for h, w in hw]
    return [W.bf16_bits_from_f32(rng.standard_normal((B, N, C, h, w)).astype(np.float32))
            for h, w in hw]


def _to_dev(a):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def _bits(t):
    t = t.detach().cpu()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).numpy()
    return t.view(torch.int32).numpy()


def _obits(a):
    return a.view(np.int16) if a.dtype in (np.uint16, np.float16) else a.view(np.int32)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_pack_and_unpack_bit_exact(case, dtype):
    import view_deformable_feature_amd as vdf
    name, B, N, C, hw = case
    say(f"[pack] {name} {dtype}")
    maps = _maps_np(name, B, N, C, hw, dtype)
    ref, rshape, rstart = oracle.pack_levels(maps)
    dmaps = [_to_dev(m) for m in maps]
    packed = vdf.da_pack_levels(dmaps)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(packed), _obits(ref))
    shape, start, nf = vdf.pack_layout(hw, N)
    assert np.array_equal(shape, rshape) and np.array_equal(start, rstart)
    # inverse, into garbage-filled outputs
    outs = [torch.full_like(m, 7.0) for m in dmaps]
    vdf.da_unpack_levels(_to_dev(ref), hw, N, out=outs)
    torch.cuda.synchronize()
    for m, o in zip(maps, outs):
        assert np.array_equal(_bits(o), _obits(m))


def test_feature_maps_format_round_trip_and_empty_batch():
    import view_deformable_feature_amd as vdf
    maps = [_to_dev(m) for m in _maps_np("fmf", 2, 3, 16, [(6, 10), (3, 5)], "f32")]
    packed, shape, start = vdf.feature_maps_format(maps)
    back = vdf.feature_maps_format([packed, shape, start], inverse=True)
    torch.cuda.synchronize()
    for m, b in zip(maps, back):
        assert torch.equal(m, b)
    empty = [torch.zeros((0, 3, 16, 6, 10), device="cuda"), torch.zeros((0, 3, 16, 3, 5), device="cuda")]
    p0 = vdf.da_pack_levels(empty)
    assert p0.shape == (0, 3 * 75, 16)


def test_gradients_through_packing():
    """maps -> pack -> aggregation: the maps' gradients are the oracle's feature
    gradient unpacked (packing is linear and its adjoint is unpacking)."""
    import view_deformable_feature_amd as vdf
    wl = W.custom("packgrad", bs=2, num_cams=3, levels=((12, 20), (6, 10)), C=64, groups=4,
                  anchors=15, pts=5, loc_lo=-0.1, loc_hi=1.1, seed=31)
    inp = W.make_inputs(wl)
    feat = inp["feat"]                                        # [bs, num_feat, C], camera-major
    hw = list(wl.levels)
    maps_np = oracle.unpack_levels(feat, hw, wl.num_cams)
    maps = [torch.from_numpy(m).cuda().requires_grad_(True) for m in maps_np]
    loc = torch.from_numpy(inp["loc"]).cuda()
    wts = torch.from_numpy(inp["weights"]).cuda()
    go = torch.from_numpy(inp["grad_out"]).cuda()
    packed, shape, start = vdf.feature_maps_format(maps)
    out = vdf.deformable_aggregation(packed, shape, start, loc, wts)
    out.backward(go)
    torch.cuda.synchronize()
    args = [inp[k] for k in KEYS]
    assert_close("packed forward", out.detach().cpu().numpy(), oracle.forward(*args), TOL_FWD)
    r_gf, _, _ = oracle.backward(*args, inp["grad_out"])
    r_maps = oracle.unpack_levels(r_gf, hw, wl.num_cams)
    for s, (m, r) in enumerate(zip(maps, r_maps)):
        assert_close(f"grad of scale {s}", m.grad.cpu().numpy(), r, TOL_BWD)
