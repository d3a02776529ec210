"""CPU oracle (test infrastructure only; never imported by the product path).

See ``oracle.attention`` for the definition it follows and how it is pinned.
"""
from .attention import (  # noqa: F401
    attend_rows,
    block_means,
    block_ranges,
    default_scale,
    dense_head,
    forward,
    forward_head,
    proxy_scores,
    route,
    route_topk,
    tile_order,
)
