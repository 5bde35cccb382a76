"""MI355X-native DiT self-attention: fused QK-RMSNorm + 3D RoPE + flash attention, dense and block-sparse,
plus the fused AdaLN update, gated residual and SwiGLU operators around it.

The compute lives in libditattn.so (HIP kernels for gfx950 behind the C ABI of
include/dit_attn.h and include/dit_block.h); this package is its thin Python binding.
"""
from ._binding import (BLOCK, DIT_ERR_HIP, DIT_ERR_HOST, DIT_ERR_INVALID_ARG, DIT_ERR_UNSUPPORTED, DIT_ERR_WORKSPACE, DIT_OK,
                       EXPORTS, HEAD_DIM, LIB_PATH, NOALLOC_SCRATCH_BYTES, DitAttnError, dit_adaln_modulate, dit_attn_block_sparse,
                       dit_attn_dense, dit_attn_dense_noalloc, dit_gated_residual, dit_swiglu,
                       dit_attn_joint, dit_attn_joint_workspace_bytes, dit_attn_keep_count, dit_attn_last_error,
                       dit_attn_route, dit_attn_set_launch_order, dit_attn_workspace_bytes, load_library,
                       workspace_for)

__all__ = ["BLOCK", "DIT_ERR_HIP", "DIT_ERR_HOST", "DIT_ERR_INVALID_ARG", "DIT_ERR_UNSUPPORTED", "DIT_ERR_WORKSPACE", "DIT_OK",
           "EXPORTS", "HEAD_DIM", "LIB_PATH", "NOALLOC_SCRATCH_BYTES", "DitAttnError", "dit_adaln_modulate", "dit_attn_block_sparse",
           "dit_attn_dense", "dit_attn_dense_noalloc", "dit_gated_residual", "dit_swiglu",
           "dit_attn_joint", "dit_attn_joint_workspace_bytes", "dit_attn_keep_count", "dit_attn_last_error",
           "dit_attn_route", "dit_attn_set_launch_order", "dit_attn_workspace_bytes", "load_library",
           "workspace_for"]
