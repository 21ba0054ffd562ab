"""Routed-expert FFN (qwen3_5-MoE shaped, low-bit affine experts) on one MI355X.

The hot path is HIP for gfx950 inside libmoe.so (C ABI in include/moe.h);
`binding` marshals torch tensors into it.
"""
from . import binding  # noqa: F401
from .binding import (  # noqa: F401
    MoeError, layer_desc, pack_layer, pack_layer_host, pack_size, route, experts,
    experts_decode, experts_grouped, workspace_size,
)
