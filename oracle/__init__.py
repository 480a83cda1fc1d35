"""Plain float64 CPU oracle for routed block-sparse attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (no kernels, headers, helpers or tables) and imports nothing from it;
it is written directly from the source pages:

* "VSA 实现详解：三维分块、均值路由与块稀疏 Attention" (maple.link) -- 3D tiling,
  per-block mean pooling, the routing matrix, TopK with a keep budget, the
  index-table format, exact sparse attention over the selected blocks, the
  coarse pooled-V branch and the H3 multi-region layout with grouped routing.
* "NSA 算子解析（Torch/Tilelang）" (devpress.csdn.net) -- the selected-attention
  branch with externally supplied block indices/counts and GQA.
* "MSA 为什么采用 KV-outer Sparse Attention Forward" (notes.kuangjux.top) -- the
  K1 local partials and the exact LSE combine of the KV-outer schedule.
* "深度解读|Spark-H3：从注意力几何到稀疏内核代码" (jefxiong.cn) -- the
  Spark-Reweight block summaries and the joint softmax of exact tokens and
  virtual tokens; the Spark-Reblock cross-moment metric and equal-capacity
  hierarchical split.

Every function computes the plain definition in float64 with NumPy: no online
softmax, no blocking, no reverse index.  The one exception is
``kv_schedule``: a plain host C++ reference of the KV-outer reverse index and
scheduler (integer work, built with g++; the tests compare the library's index
with it exactly and run its brute-force checker under the address and
undefined-behaviour sanitizers).  Each one is pinned by the ``not gpu``
tests in ``tests/test_oracle_*.py`` against values printed on the pages,
closed forms, brute force and library routines.
"""

from .tiling import tile_dims, tile_index, keep_budget
from .routing import pool_blocks, routing_matrix, select_topk
from .attention import (
    vsa_attention,
    nsa_attention,
    kvouter_partials,
    lse_combine,
)
from .reweight import anchor_queries, block_summaries, virtual_logit, reweight_attention
from .coarse import coarse_attention, add_coarse
from .h3 import h3_layout, h3_route
from . import reblock

__all__ = [
    "h3_layout",
    "h3_route",
    "reblock",
    "tile_dims",
    "tile_index",
    "keep_budget",
    "pool_blocks",
    "routing_matrix",
    "select_topk",
    "vsa_attention",
    "anchor_queries",
    "block_summaries",
    "virtual_logit",
    "reweight_attention",
    "coarse_attention",
    "add_coarse",
    "nsa_attention",
    "kvouter_partials",
    "lse_combine",
]
