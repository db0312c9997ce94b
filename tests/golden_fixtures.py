"""Loader for the hand-derived fixtures under ``tests/golden/``.

Each fixture is a JSON file with a citation of the passage it follows, the
derivation of its expected values by hand, the inputs, and the expected
outputs.  No expected value in them was produced by running code.
"""
import glob
import json
import os

import numpy as np

GOLDEN_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _with_keys(*keys):
    out = []
    for p in sorted(glob.glob(os.path.join(GOLDEN_DIR, "*.json"))):
        with open(p) as f:
            d = json.load(f)
        if all(k in d for k in keys):
            out.append(p)
    return out


def fixture_paths():
    """The deformable-aggregation fixtures (features, locations, weights)."""
    return _with_keys("feat", "loc", "weights")


def dcn_fixture_paths():
    """The deformable-convolution fixtures (input, offset_mask)."""
    return _with_keys("input", "offset_mask")


def load(path):
    with open(path) as f:
        d = json.load(f)
    inp = dict(
        feat=np.asarray(d["feat"], dtype=np.float32),
        spatial_shape=np.asarray(d["spatial_shape"], dtype=np.int32),
        scale_start_index=np.asarray(d["scale_start_index"], dtype=np.int32),
        loc=np.asarray(d["loc"], dtype=np.float32),
        weights=np.asarray(d["weights"], dtype=np.float32),
        grad_out=np.asarray(d["grad_out"], dtype=np.float32),
    )
    exp = {k[len("expect_"):]: np.asarray(v, dtype=np.float64)
           for k, v in d.items() if k.startswith("expect_")}
    return d, inp, exp
