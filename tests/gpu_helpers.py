"""Helpers shared by the GPU tests: run the HIP path through the C ABI on
seeded inputs and compare with the oracle element by element.

Tolerances (per element, |gpu - ref| <= tol * (1 + |ref|)):
  forward, binary32 features        1e-4
  backward (atomic sums), binary32  1e-3
  bfloat16 features                 1e-2
  binary16 features                 as binary32 (they convert exactly)
  out stored in bfloat16 / binary16 the forward bound plus the rounding of one
                                    result: 2^-8 / 2^-11 of |ref|
"""
import sys

import numpy as np
import torch

TOL_FWD = 1e-4
TOL_BWD = 1e-3
TOL_BF16 = 1e-2
TOL_OUT_BF16 = TOL_FWD + 2.0 ** -8
TOL_OUT_F16 = TOL_FWD + 2.0 ** -11

KEYS = ("feat", "spatial_shape", "scale_start_index", "loc", "weights")


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(inp, device="cuda"):
    d = {}
    feat = inp["feat"]
    if feat.dtype == np.uint16:
        d["feat"] = torch.from_numpy(feat.view(np.int16)).to(device).view(torch.bfloat16)
    else:
        d["feat"] = torch.from_numpy(feat).to(device)
    for k in ("loc", "weights", "grad_out"):
        if k in inp:
            d[k] = torch.from_numpy(np.ascontiguousarray(inp[k])).to(device)
    d["spatial_shape"] = inp["spatial_shape"]
    d["scale_start_index"] = inp["scale_start_index"]
    return d


def gpu_forward(dev, slices=None, workspace=None, out_dtype=None):
    """slices: None = the library's choice, True / False = level slices forced on / off."""
    import view_deformable_feature_amd as vdf
    out = vdf.da_forward(dev["feat"], dev["spatial_shape"], dev["scale_start_index"],
                         dev["loc"], dev["weights"], workspace=workspace, slices=slices,
                         out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out


def gpu_backward(dev, accumulate_into=None, atomic=False, workspace=None, slices=None,
                 regather=None, deterministic=False):
    """regather: None = the library's choice of backward form, True = per-anchor,
    False = row-ordered."""
    import view_deformable_feature_amd as vdf
    args = (dev["feat"], dev["spatial_shape"], dev["scale_start_index"], dev["loc"],
            dev["weights"], dev["grad_out"])
    if atomic:
        r = vdf.da_backward_atomic(*args)
    elif accumulate_into is None:
        r = vdf.da_backward(*args, workspace=workspace, slices=slices, regather=regather,
                            deterministic=deterministic)
    else:
        r = vdf.da_backward_accumulate(*args, accumulate_into, workspace=workspace,
                                       slices=slices, regather=regather,
                                       deterministic=deterministic)
    torch.cuda.synchronize()
    return r


def assert_close(name, got, ref, tol):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, f"{name}: shape {got.shape} vs {ref.shape}"
    err = np.abs(got - ref)
    bound = tol * (1.0 + np.abs(ref))
    bad = ~(err <= bound)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        rows = [(tuple(i), got[tuple(i)], ref[tuple(i)]) for i in idx]
        raise AssertionError(f"{name}: {int(bad.sum())} of {bad.size} elements exceed "
                             f"tol {tol}; max err {err.max():.3e}; first: {rows}")
    return float(err.max()) if err.size else 0.0
