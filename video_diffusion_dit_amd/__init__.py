"""MI355X-native (gfx950) BF16 attention forward for video-diffusion DiTs.

The compute lives in ``lib/libattn.so`` (hand-written HIP kernels behind the C ABI of
``include/attn.h``); ``attention`` is its thin torch binding. Importing this package does
not load the library; the first call does, and raises if it has not been built.
"""
from .attention import (AttnError, attn_fwd, attn_fwd_block_sparse, attn_fwd_block_sparse_varlen, attn_fwd_varlen,
                        attn_fwd_varlen_noalloc,
                        block_list_stride, block_route, block_route_varlen, block_skip_attention,
                        block_skip_attention_varlen, block_skip_use_dense,
                        check_cu_seqlens, linear_attention, load_library, qk_norm_packed, qk_prologue, splitkv_workspace_bytes,
                        try_attn_fwd, varlen_list_shapes, varlen_tile_offsets, varlen_workspace_bytes)

__all__ = ["AttnError", "attn_fwd", "attn_fwd_block_sparse", "attn_fwd_block_sparse_varlen", "attn_fwd_varlen",
           "attn_fwd_varlen_noalloc",
           "block_list_stride", "block_route", "block_route_varlen", "block_skip_attention",
           "block_skip_attention_varlen", "block_skip_use_dense",
           "check_cu_seqlens", "linear_attention", "load_library", "qk_norm_packed", "qk_prologue",
           "splitkv_workspace_bytes",
           "try_attn_fwd", "varlen_list_shapes", "varlen_tile_offsets", "varlen_workspace_bytes"]
