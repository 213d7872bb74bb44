"""int4 expert-routed MoE layer for AMD MI355X: Python binding over libmoe_q4.so.

The HIP kernels and the C ABI live in csrc/ and include/moe_q4.h; this package
only loads the library and marshals torch tensors into it.
"""
from . import ops  # noqa: F401
from .ops import (  # noqa: F401
    MoELayer,
    MoEWeights,
    Q4Stack,
    max_tiles,
    moe_grouped_gemm_q4,
    moe_layer_forward,
    moe_route,
    workspace_bytes,
)
