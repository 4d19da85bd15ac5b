"""MI355X-native MoE expert layer: routing, sentinel-aware offsets, permute,
grouped GEMMs with fused SiLU*up, and combine (and the layer's backward), as
hand-written HIP for gfx950
behind the C ABI in ``include/moe.h``.

``ops`` holds torch-tensor wrappers (argument marshalling only); ``_lib``
loads ``libmoe.so``; ``build`` compiles it.
"""

from ._lib import MoeKernels, load  # noqa: F401
from .ops import (  # noqa: F401
    Gradients,
    backward,
    backward_workspace_bytes,
    build_offsets,
    build_offsets_noalloc,
    forward,
    forward_workspace_bytes,
    grouped_gemm,
    grouped_gemm_gather,
    grouped_gemm_tile_shape,
    permute,
    quantize_rows,
    route_topk,
    unpermute_combine,
)
