"""Routed block-sparse attention for AMD Instinct MI355X (gfx950).

The hot path lives in libbsa.so (hand-written HIP kernels behind the C ABI of
include/bsa.h); this package is a thin PyTorch binding over it.  Importing the
package loads the library and raises if it has not been built -- there is no
fallback implementation.
"""

from . import _lib
from .api import (
    tile_dims,
    tile_index,
    keep_budget,
    pool_route_topk,
    route_workspace_bytes,
    attention_vsa,
    coarse_attention,
    spark_summaries,
    attention_nsa,
    kvouter,
    combine,
    VsaGeometry,
    vsa_forward,
    H3Geometry,
    h3_pool_route_topk,
    h3_forward,
    spark_reblock,
    reblock_forward,
    qouter_workspace,
    check,
)
from . import metrics

_lib.load()

__all__ = [
    "tile_dims",
    "tile_index",
    "keep_budget",
    "pool_route_topk",
    "route_workspace_bytes",
    "attention_vsa",
    "coarse_attention",
    "spark_summaries",
    "attention_nsa",
    "kvouter",
    "combine",
    "VsaGeometry",
    "vsa_forward",
    "H3Geometry",
    "h3_pool_route_topk",
    "h3_forward",
    "spark_reblock",
    "reblock_forward",
    "qouter_workspace",
    "check",
    "metrics",
]
