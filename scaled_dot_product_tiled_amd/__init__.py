"""libattn: fused causal grouped-query attention for AMD MI355X (gfx950).

The computation lives in HIP kernels behind a C ABI (include/attn.h, built into
libattn.so by ``scaled_dot_product_tiled_amd.build``); this package only marshals
torch tensors into those calls.
"""
from .binding import attn_bwd, attn_fwd, load_library, paged_decode  # noqa: F401

__all__ = ["attn_fwd", "attn_bwd", "paged_decode", "load_library"]
