"""libattn: fused causal grouped-query attention for AMD MI355X (gfx950).

The computation lives in HIP kernels behind a C ABI (include/attn.h, built into
libattn.so by ``scaled_dot_product_tiled_amd.build``); this package only marshals
torch tensors into those calls.
"""
from .binding import (DecodeGraphs, attn_bwd, attn_bwd_chunk, attn_bwd_chunk_workspace_bytes, attn_fwd, attn_fwd_chunk,  # noqa: F401
                      attn_fwd_chunk_merge, attn_fwd_paged, attn_fwd_paged_split, attn_lse_merge, debug, load_library, paged_decode,
                      paged_decode_contiguous, paged_decode_noalloc, paged_kv_append, paged_kv_gather)

__all__ = ["DecodeGraphs", "attn_fwd", "attn_bwd", "attn_fwd_chunk", "attn_bwd_chunk", "attn_bwd_chunk_workspace_bytes",
           "attn_lse_merge", "attn_fwd_chunk_merge", "attn_fwd_paged", "attn_fwd_paged_split", "paged_decode", "paged_decode_contiguous",
           "paged_decode_noalloc",
           "paged_kv_append", "paged_kv_gather", "debug", "load_library"]
