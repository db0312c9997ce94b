"""Pins of the oracle's level packing (section 6 of the Sparse4D walkthrough,
feature_maps_format; layout of section 3.1): an explicit loop over every
element, agreement with the workload generator's level table, the inverse,
and the level table the library computes on the host."""
import numpy as np
import pytest

import oracle
from view_deformable_feature_amd import workloads as W


def _maps(rng, B, N, C, hw, dtype=np.float32):
    return [rng.standard_normal((B, N, C, h, w)).astype(dtype) for h, w in hw]


def test_pack_matches_elementwise_definition():
    rng = np.random.default_rng(3)
    hw = [(3, 5), (2, 2), (1, 3)]
    maps = _maps(rng, 2, 3, 4, hw)
    packed, shape, start = oracle.pack_levels(maps)
    assert packed.shape == (2, 3 * (15 + 4 + 3), 4)
    seen = np.zeros(packed.shape, bool)
    for b in range(2):
        for k in range(3):
            for s, (h, w) in enumerate(hw):
                assert tuple(shape[k, s]) == (h, w)
                for i in range(h):
                    for j in range(w):
                        for c in range(4):
                            r = start[k, s] + i * w + j
                            assert packed[b, r, c] == maps[s][b, k, c, i, j]
                            seen[b, r, c] = True
    assert seen.all()                      # every packed element comes from a map element
    # camera-major: camera k's block starts after k full pyramids
    assert list(start[:, 0]) == [0, 22, 44]
    assert list(start[1]) == [22, 37, 41]


def test_pack_layout_is_the_generators_level_table():
    wl = W.WORKLOADS["nuscenes_fwd"]
    shape, start = W.level_table(wl)
    maps = [np.zeros((1, wl.num_cams, 1, h, w), np.float32) for h, w in wl.levels]
    _, pshape, pstart = oracle.pack_levels(maps)
    assert np.array_equal(shape, pshape) and np.array_equal(start, pstart)


def test_unpack_inverts_pack():
    rng = np.random.default_rng(4)
    hw = [(7, 9), (4, 5), (1, 1)]
    maps = _maps(rng, 2, 2, 3, hw)
    packed, _, _ = oracle.pack_levels(maps)
    back = oracle.unpack_levels(packed, hw, 2)
    for m, r in zip(maps, back):
        assert np.array_equal(m, r)
    # and pack(unpack(x)) == x for an arbitrary packed tensor
    x = rng.standard_normal(packed.shape).astype(np.float32)
    assert np.array_equal(oracle.pack_levels(oracle.unpack_levels(x, hw, 2))[0], x)


def test_library_layout_matches_oracle():
    import view_deformable_feature_amd as vdf
    from view_deformable_feature_amd.build import build, is_stale
    if is_stale():
        build()
    hw = [(64, 176), (32, 88), (16, 44), (8, 22)]
    maps = [np.zeros((1, 6, 1, h, w), np.float32) for h, w in hw]
    _, oshape, ostart = oracle.pack_levels(maps)
    shape, start, nf = vdf.pack_layout(hw, 6)
    assert np.array_equal(shape, oshape) and np.array_equal(start, ostart) and nf == 89760


@pytest.mark.parametrize("kw, needle", [
    (dict(scale_hw=[(0, 4)]), "outside [1"),
    (dict(scale_hw=[(4, 40000)]), "outside [1"),
    (dict(num_cams=0), ">= 1"),
    (dict(num_cams=9, scale_hw=[(2, 2)] * 8), "DA_MAX_LEVELS"),
])
def test_library_layout_rejects_malformed(kw, needle):
    import view_deformable_feature_amd as vdf
    from view_deformable_feature_amd._lib import DAError
    args = dict(scale_hw=[(4, 4)], num_cams=2)
    args.update(kw)
    with pytest.raises(DAError, match=needle.replace("[", r"\[")):
        vdf.pack_layout(args["scale_hw"], args["num_cams"])
