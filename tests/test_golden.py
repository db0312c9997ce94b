"""The oracle reproduces the hand-derived worked examples in ``tests/golden/``."""
import os

import numpy as np
import pytest

import oracle
from golden_fixtures import fixture_paths, load

KEYS = ("feat", "spatial_shape", "scale_start_index", "loc", "weights")


@pytest.mark.parametrize("path", fixture_paths(), ids=os.path.basename)
def test_oracle_matches_hand_derivation(path):
    d, inp, exp = load(path)
    assert d["citation"] and d["derivation"]
    args = [inp[k] for k in KEYS]
    np.testing.assert_allclose(oracle.forward(*args), exp["out"], rtol=0, atol=1e-15)
    gf, gl, gw = oracle.backward(*args, inp["grad_out"])
    np.testing.assert_allclose(gf, exp["grad_feat"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(gl, exp["grad_loc"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(gw, exp["grad_weights"], rtol=0, atol=1e-15)


def test_fixtures_present():
    assert len(fixture_paths()) >= 2
