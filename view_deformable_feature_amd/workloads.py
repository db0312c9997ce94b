"""Seeded synthetic workloads for deformable aggregation.

This module only draws random inputs; it holds none of the operator's
arithmetic.  Both the HIP path and the fp64 oracle consume the arrays it
returns, byte for byte, so the two sides always see identical inputs.

Shapes follow the multi-camera, multi-scale setting of the Sparse4D
deformable_aggregation walkthrough (mhpn.cn/news/1081857), sections 5.1
(the six work dimensions) and 6 (``DeformableAggregationFunction`` inputs):

  mc_ms_feat         [bs, num_feat, C]        HWC rows of every (camera, scale) level
  spatial_shape      [num_cams, num_scale, 2] int32 (H, W) of each level
  scale_start_index  [num_cams, num_scale]    int32 first row of each level
  sampling_location  [bs, A, P, K, 2]         float32 normalised (x, y)
  weights            [bs, A, P, K, S, G]      float32
  grad_out           [bs, A, C]               float32

Levels are stored camera-major, scale-minor, each level row-major (H, W)
with C contiguous channels.  Draw order per workload is fixed: features,
locations, weights, grad_out, all from ``numpy.random.default_rng(seed)``.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Tuple

import numpy as np

__all__ = ["Workload", "WORKLOADS", "make_inputs", "bf16_bits_from_f32",
           "bf16_bits_to_f32", "level_table", "DcnWorkload", "DCN_WORKLOADS",
           "make_dcn_inputs", "dcn_custom"]


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic configuration of the operator.

    ``levels`` gives (H, W) per scale; every camera has the same pyramid
    unless ``cam_levels`` overrides it with one tuple of (H, W) per camera.
    """
    name: str
    bs: int
    num_cams: int
    levels: Tuple[Tuple[int, int], ...]
    C: int
    groups: int
    anchors: int
    pts: int
    feat_dtype: str = "f32"            # "f32", "bf16" or "f16"
    loc_kind: str = "uniform"          # "uniform" or "clustered"
    loc_lo: float = 0.0
    loc_hi: float = 1.0
    loc_sigma: float = 0.02
    weight_kind: str = "softmax"       # "softmax" or "uniform01"
    seed: int = 0
    cam_levels: Optional[Tuple[Tuple[Tuple[int, int], ...], ...]] = None

    @property
    def num_scale(self) -> int:
        return len(self.levels)

    def level_hw(self) -> List[List[Tuple[int, int]]]:
        if self.cam_levels is not None:
            assert len(self.cam_levels) == self.num_cams
            return [list(c) for c in self.cam_levels]
        return [list(self.levels) for _ in range(self.num_cams)]

    @property
    def num_feat(self) -> int:
        return sum(h * w for cam in self.level_hw() for (h, w) in cam)

    @property
    def num_samples(self) -> int:
        """bs * A * P * K * S bilinear samples per pass."""
        return self.bs * self.anchors * self.pts * self.num_cams * self.num_scale

    @property
    def sample_channels(self) -> int:
        return self.num_samples * self.C

    @property
    def feat_elem_bytes(self) -> int:
        return 2 if self.feat_dtype in ("bf16", "f16") else 4


_NUSC_LEVELS = ((64, 176), (32, 88), (16, 44), (8, 22))      # 256x704 image, strides 4..32
_LARGE_LEVELS = ((160, 400), (80, 200), (40, 100), (20, 50))  # 640x1600 image, strides 4..32

WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", bs=1, num_cams=1, levels=((16, 16),), C=32, groups=1,
                     anchors=8, pts=4, loc_lo=-0.1, loc_hi=1.1,
                     weight_kind="uniform01", seed=1000),
    "nuscenes_fwd": Workload("nuscenes_fwd", bs=1, num_cams=6, levels=_NUSC_LEVELS, C=256,
                             groups=8, anchors=900, pts=13, loc_lo=-0.05, loc_hi=1.05,
                             seed=1001),
    "nuscenes_bwd": Workload("nuscenes_bwd", bs=1, num_cams=6, levels=_NUSC_LEVELS, C=256,
                             groups=8, anchors=900, pts=13, loc_lo=-0.05, loc_hi=1.05,
                             seed=1002),
    "large": Workload("large", bs=4, num_cams=6, levels=_LARGE_LEVELS, C=256, groups=8,
                      anchors=1500, pts=13, loc_kind="clustered", loc_sigma=0.02,
                      seed=1003),
    "large_bf16": Workload("large_bf16", bs=4, num_cams=6, levels=_LARGE_LEVELS, C=256,
                           groups=8, anchors=1500, pts=13, feat_dtype="bf16",
                           loc_lo=0.0, loc_hi=1.0, seed=1004),
    # the nuScenes shape with binary16 features (half precision, as DCNv4 runs)
    "nuscenes_f16": Workload("nuscenes_f16", bs=1, num_cams=6, levels=_NUSC_LEVELS, C=256,
                             groups=8, anchors=900, pts=13, feat_dtype="f16",
                             loc_lo=-0.05, loc_hi=1.05, seed=1005),
}


def level_table(wl: Workload) -> Tuple[np.ndarray, np.ndarray]:
    """(spatial_shape [K,S,2] int32, scale_start_index [K,S] int32), camera-major."""
    hw = wl.level_hw()
    shape = np.zeros((wl.num_cams, wl.num_scale, 2), dtype=np.int32)
    start = np.zeros((wl.num_cams, wl.num_scale), dtype=np.int32)
    row = 0
    for k in range(wl.num_cams):
        assert len(hw[k]) == wl.num_scale
        for s, (h, w) in enumerate(hw[k]):
            shape[k, s] = (h, w)
            start[k, s] = row
            row += h * w
    return shape, start


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the raw 16-bit patterns as uint16.  Inputs are finite draws.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    out = np.empty(u.shape, dtype=np.uint16)
    chunk = 1 << 24
    flat_u, flat_o = u.reshape(-1), out.reshape(-1)
    for i in range(0, flat_u.size, chunk):
        v = flat_u[i:i + chunk]
        lsb = (v >> np.uint32(16)) & np.uint32(1)
        flat_o[i:i + chunk] = ((v + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _softmax_weights(rng: np.random.Generator, wl: Workload) -> np.ndarray:
    """Aggregation weights that sum to one over (P, K, S) for each (b, a, g)."""
    bs, A, P, K, S, G = wl.bs, wl.anchors, wl.pts, wl.num_cams, wl.num_scale, wl.groups
    out = np.empty((bs, A, P, K, S, G), dtype=np.float32)
    for b in range(bs):  # one batch at a time keeps the float64 temporaries small
        logits = rng.standard_normal((A, P * K * S, G))
        logits -= logits.max(axis=1, keepdims=True)
        e = np.exp(logits)
        e /= e.sum(axis=1, keepdims=True)
        out[b] = e.reshape(A, P, K, S, G).astype(np.float32)
    return out


def make_inputs(wl: Workload, seed: Optional[int] = None, with_grad_out: bool = True
                ) -> Dict[str, np.ndarray]:
    """Draw one batch of inputs for ``wl``.

    Returns a dict with ``feat`` (float32; uint16 bf16 bit patterns when
    ``wl.feat_dtype == "bf16"``; float16 when "f16"), ``spatial_shape``, ``scale_start_index``,
    ``loc``, ``weights`` and (optionally) ``grad_out``.
    """
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    bs, A, P, K, S, G, C = (wl.bs, wl.anchors, wl.pts, wl.num_cams, wl.num_scale,
                            wl.groups, wl.C)
    shape, start = level_table(wl)
    feat = rng.standard_normal((bs, wl.num_feat, C), dtype=np.float32)
    if wl.feat_dtype == "bf16":
        feat = bf16_bits_from_f32(feat)
    elif wl.feat_dtype == "f16":
        feat = feat.astype(np.float16)           # round to nearest even
    elif wl.feat_dtype != "f32":
        raise ValueError(f"unknown feat dtype {wl.feat_dtype!r}")

    if wl.loc_kind == "uniform":
        loc = rng.uniform(wl.loc_lo, wl.loc_hi, size=(bs, A, P, K, 2)).astype(np.float32)
    elif wl.loc_kind == "clustered":
        centre = rng.random((bs, A, 1, K, 2))
        loc = (centre + rng.normal(0.0, wl.loc_sigma, size=(bs, A, P, K, 2))).astype(np.float32)
    else:
        raise ValueError(f"unknown loc kind {wl.loc_kind!r}")

    if wl.weight_kind == "softmax":
        weights = _softmax_weights(rng, wl)
    elif wl.weight_kind == "uniform01":
        weights = rng.random((bs, A, P, K, S, G), dtype=np.float32)
    else:
        raise ValueError(f"unknown weight kind {wl.weight_kind!r}")

    out = dict(feat=feat, spatial_shape=shape, scale_start_index=start, loc=loc,
               weights=weights)
    if with_grad_out:
        out["grad_out"] = rng.standard_normal((bs, A, C), dtype=np.float32)
    return out


def custom(name: str, **kw) -> Workload:
    """A workload with explicit fields (used by tests for ragged shapes)."""
    return Workload(name=name, **kw)


# ---------------------------------------------------------------------------------------
# deformable convolution (DCNv3 / DCNv4 operator) inputs
# ---------------------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class DcnWorkload:
    """Shapes of one deformable-convolution call: input [N, H, W, C] channel-last,
    offset_mask [N, Ho, Wo, G, 3K] ((dx, dy) per tap, then the K modulation scalars)."""
    name: str
    N: int
    H: int
    W: int
    C: int
    groups: int
    kernel: Tuple[int, int] = (3, 3)
    stride: Tuple[int, int] = (1, 1)
    pad: Tuple[int, int] = (1, 1)
    dilation: Tuple[int, int] = (1, 1)
    dtype: str = "f32"                 # "f32", "bf16" or "f16"
    offset_sigma: float = 1.0          # offsets N(0, sigma^2) pixels
    seed: int = 0

    @property
    def K(self) -> int:
        return self.kernel[0] * self.kernel[1]

    @property
    def out_hw(self) -> Tuple[int, int]:
        ho = (self.H + 2 * self.pad[0] - self.dilation[0] * (self.kernel[0] - 1) - 1) // self.stride[0] + 1
        wo = (self.W + 2 * self.pad[1] - self.dilation[1] * (self.kernel[1] - 1) - 1) // self.stride[1] + 1
        return ho, wo

    @property
    def samples(self) -> int:
        """bilinear samples per call: N * Ho * Wo * G * K"""
        ho, wo = self.out_hw
        return self.N * ho * wo * self.groups * self.K

    @property
    def sample_channels(self) -> int:
        return self.samples * (self.C // self.groups)

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


# The DCNv4 notes time the operator at 56x56x128 with batch 64 and 4 groups (its
# kernel ablation table) and compare input sizes 28x28x256 and 14x14x512 (its first
# figure; groups not stated there: 32 channels per group kept).
DCN_WORKLOADS: Dict[str, DcnWorkload] = {
    "dcn_tiny": DcnWorkload("dcn_tiny", N=1, H=7, W=9, C=16, groups=2, seed=2000),
    "dcn_56": DcnWorkload("dcn_56", N=64, H=56, W=56, C=128, groups=4, seed=2001),
    "dcn_56_f16": DcnWorkload("dcn_56_f16", N=64, H=56, W=56, C=128, groups=4, dtype="f16",
                              seed=2002),
    "dcn_28": DcnWorkload("dcn_28", N=64, H=28, W=28, C=256, groups=8, seed=2003),
    "dcn_14": DcnWorkload("dcn_14", N=64, H=14, W=14, C=512, groups=16, seed=2004),
}


def make_dcn_inputs(wl: DcnWorkload, seed: Optional[int] = None, with_grad_out: bool = True
                    ) -> Dict[str, np.ndarray]:
    """Draw one call's inputs: ``input`` (float32, float16, or uint16 bfloat16 bit
    patterns), ``offset_mask`` (offsets N(0, sigma^2) pixels, scalars U[-1, 1): DCNv4
    leaves them unbounded) and ``grad_out`` N(0, 1)."""
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    ho, wo = wl.out_hw
    x = rng.standard_normal((wl.N, wl.H, wl.W, wl.C), dtype=np.float32)
    if wl.dtype == "bf16":
        x = bf16_bits_from_f32(x)
    elif wl.dtype == "f16":
        x = x.astype(np.float16)
    elif wl.dtype != "f32":
        raise ValueError(f"unknown dtype {wl.dtype!r}")
    G, K = wl.groups, wl.K
    om = np.empty((wl.N, ho, wo, G, 3 * K), dtype=np.float32)
    om[..., :2 * K] = rng.normal(0.0, wl.offset_sigma, size=(wl.N, ho, wo, G, 2 * K))
    om[..., 2 * K:] = rng.uniform(-1.0, 1.0, size=(wl.N, ho, wo, G, K))
    out = dict(input=x, offset_mask=om)
    if with_grad_out:
        out["grad_out"] = rng.standard_normal((wl.N, ho, wo, wl.C), dtype=np.float32)
    return out


def dcn_custom(name: str, **kw) -> DcnWorkload:
    return DcnWorkload(name=name, **kw)
