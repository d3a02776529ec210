"""On-the-fly block-sparse self-attention for video DiTs on MI355X (gfx950).

The compute path is the HIP library libsa_route.so (C ABI in include/sa_route.h);
``block_sparse_attention_route_amd.api`` is its Python binding and
``block_sparse_attention_route_amd.synth`` generates seeded synthetic inputs.
"""
from . import api  # noqa: F401
from .api import (  # noqa: F401
    SaError,
    sa_dense_forward,
    sa_forward,
    sa_forward_pooled,
    sa_pool,
    sa_route,
    sa_workspace_bytes,
)
