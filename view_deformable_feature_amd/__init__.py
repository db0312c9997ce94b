"""Sparse4D-style deformable aggregation for AMD Instinct MI355X (gfx950).

The computation lives in ``libdeformagg.so`` (HIP kernels behind a C ABI,
declared in ``include/deformagg.h`` and ``include/dcn.h``); ``api``, ``pack`` and
``dcn`` bind it to PyTorch tensors.
``workloads`` draws seeded synthetic inputs.
"""
from .api import (DeformableAggregationFunction, da_backward, da_backward_accumulate,  # noqa: F401
                  da_backward_atomic, da_forward, deformable_aggregation, forward_workspace_size,
                  workspace_size)

from .pack import (PackLevelsFunction, da_pack_levels, da_unpack_levels,  # noqa: F401
                   feature_maps_format, pack_layout, pack_levels)

from .dcn import (DCNFunction, dcn_backward, dcn_forward, dcn_out_size,  # noqa: F401
                  dcn_workspace_size, deformable_conv)

__version__ = "1.2.0"
