"""MI355X (gfx950) MoE token routing layout, dispatch and combine (layout and
dispatch also fused into two launches: MoeDispatcher.layout_dispatch), their
backward, and the expert step between them (a grouped GEMM driven by the
device-side offsets).

The compute lives in libmoe_layout.so (hand-written HIP kernels behind the C
ABI of include/moe.h); this package is its thin Python binding.
"""
from .moe import (  # noqa: F401
    Dispatched, Layout, MoeDispatcher, TiledExpertWeights, ceil_div, grouped_gemm,
    layout_noalloc, num_max_tokens_infer, num_max_tokens_pretrain, round_up4,
    tile_expert_weights, validate_num_max,
)
from ._lib import MoeError, load  # noqa: F401
from .autograd import MoeTokenDispatcher  # noqa: F401
